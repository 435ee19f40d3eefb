"""moe_forward_static (the whole layer with its workspace in a static device
array, for callers that cannot allocate) against moe_forward with a caller
workspace: the same kernels on the same inputs, so outputs, expert indices and
weights must be equal bit for bit.  Two calls in a row on each layer, the second
with fewer tokens, so the second call runs on the array the first one left
behind."""
import numpy as np
import pytest
import torch

from parity import say
from routed_expert_moe_amd import binding as B
from routed_expert_moe_amd import configs, synth
from routed_expert_moe_amd.configs import LayerShape

pytestmark = pytest.mark.gpu

CASES = {
    # fp8 weight-streaming path (16-row tiles)
    "v3_decode_fp8": (configs.V3_DECODE_FP8.with_(name="static_v3_decode", T=16), (16, 5)),
    # bf16 MFMA path with the expert-chunk GEMM, groups, bias and a shared expert
    "mfma_groups": (LayerShape(
        name="static_mfma_groups", T=777, dim=384, n_routed=32, n_groups=4, topk_groups=2, top_k=4,
        n_shared=1, inter_dim=320, score="sigmoid", route_scale=2.5, act="bf16", weight="bf16",
        seed=61, bias_range=0.1), (777, 300)),
    # fp32 SIMT path
    "tiny_f32": (configs.TINY_F32, (64, 37)),
}


def _layer(shape):
    dev = "cpu" if shape.T * shape.dim * shape.n_routed < 2 ** 27 else "cuda"
    lay = synth.make_layer(shape, device=dev)
    if dev == "cpu":
        for f in ("x", "w_gate", "bias", "w13", "w2", "sw13", "sw2", "w13_scale", "w2_scale",
                  "sw13_scale", "sw2_scale"):
            t = getattr(lay, f)
            if t is not None:
                setattr(lay, f, t.cuda())
    return lay


@pytest.mark.parametrize("name", list(CASES))
def test_static_workspace_forward_equals_forward(name):
    shape, Ts = CASES[name]
    layer = _layer(shape)
    cfg = B.config_of(shape)
    w = B.weights_of(layer)
    K = shape.top_k
    for T in Ts:
        say(f"[moe_forward_static] {shape.name} T={T}")
        x = layer.x[:T].contiguous()
        ws = torch.empty(max(B.moe_workspace_size(cfg, T), 256), dtype=torch.uint8, device="cuda")
        out_ref = torch.empty_like(x)
        idx_ref = torch.empty(T, K, dtype=torch.int32, device="cuda")
        w_ref = torch.empty(T, K, dtype=torch.float32, device="cuda")
        B.moe_forward(cfg, T, x, w, out_ref, idx_ref, w_ref, ws)
        out = torch.full_like(x, float("nan"))
        idx = torch.full((T, K), -7, dtype=torch.int32, device="cuda")
        wt = torch.full((T, K), float("nan"), dtype=torch.float32, device="cuda")
        B.moe_forward_static(cfg, T, x, w, out, idx, wt)
        torch.cuda.synchronize()
        assert torch.equal(out, out_ref), f"{shape.name} T={T}: outputs differ"
        assert torch.equal(idx, idx_ref) and torch.equal(wt, w_ref), f"{shape.name} T={T}: routing differs"
        assert bool(torch.isfinite(out.float()).all())
        del ws


def test_static_workspace_rejects_large_layers():
    """A layer whose workspace exceeds the static array fails before any launch."""
    shape = configs.V3_PREFILL_BF16
    cfg = B.config_of(shape)
    assert B.moe_workspace_size(cfg, shape.T) > 64 << 20
    x = torch.zeros(1, device="cuda")
    with pytest.raises(B.MoeError) as ei:
        B.moe_forward_static(cfg, shape.T, x, B.moe_weights(), x)
    assert ei.value.status == B.MOE_ERR_WORKSPACE
