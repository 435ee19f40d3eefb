"""GPU parity of the FP8 W8A8 path (fp8 expert weights, activations quantised
1 x 128 to e4m3 before each expert GEMM) against the W8A8 oracle.

The quantisation of x is compared code for code and scale for scale (both
sides decide in float32 from the exact bf16 inputs).  The layer output is
compared on the GPU's expert selection within the fp8 tolerance, on h' and on
h' - u; the SwiGLU output h is quantised from each side's own fp32 value, so a
code may differ where the two straddle a rounding midpoint.
"""
import numpy as np
import pytest
import torch

from oracle import w8a8
from oracle_bridge import run_oracle, to_f64
from parity import TOL, rel_err, say
from routed_expert_moe_amd import binding as B
from routed_expert_moe_amd import configs, synth
from routed_expert_moe_amd.configs import LayerShape

pytestmark = pytest.mark.gpu

SHAPES = {
    "w8a8_small": LayerShape(
        name="w8a8_small", T=300, dim=256, n_routed=32, n_groups=4, topk_groups=2, top_k=4,
        n_shared=1, inter_dim=256, score="sigmoid", route_scale=2.5, act="bf16", weight="fp8",
        act_quant=1, seed=41, bias_range=0.05),
    "w8a8_T1": LayerShape(
        name="w8a8_T1", T=1, dim=256, n_routed=32, n_groups=4, topk_groups=2, top_k=4,
        n_shared=1, inter_dim=256, score="sigmoid", route_scale=2.5, act="bf16", weight="fp8",
        act_quant=1, seed=42, bias_range=0.05),
    "w8a8_softmax_noshared": LayerShape(
        name="w8a8_softmax_noshared", T=200, dim=384, n_routed=16, n_groups=1, topk_groups=1,
        top_k=2, n_shared=0, inter_dim=128, score="softmax", route_scale=1.0, act="bf16",
        weight="fp8", act_quant=1, seed=43),
    "w8a8_ragged_2shared": LayerShape(
        name="w8a8_ragged_2shared", T=777, dim=512, n_routed=64, n_groups=8, topk_groups=4,
        top_k=6, n_shared=2, inter_dim=384, score="sigmoid", route_scale=2.5, act="bf16",
        weight="fp8", act_quant=1, seed=44, bias_range=0.05),
    "v3_decode_w8a8": configs.V3_DECODE_FP8.with_(name="v3_decode_w8a8_T8", act_quant=1),
}


def _layer(shape):
    dev = "cpu" if shape.T * shape.dim * shape.n_routed < 2 ** 27 else "cuda"
    say(f"[make_layer] {shape.name} T={shape.T} seed={shape.seed}")
    lay = synth.make_layer(shape, device=dev)
    if dev == "cpu":
        for f in ("x", "w_gate", "bias", "w13", "w2", "sw13", "sw2", "w13_scale", "w2_scale",
                  "sw13_scale", "sw2_scale"):
            t = getattr(lay, f)
            if t is not None:
                setattr(lay, f, t.cuda())
    return lay


@pytest.mark.parametrize("shape", [SHAPES["w8a8_small"], SHAPES["w8a8_ragged_2shared"],
                                   configs.V3_PREFILL_W8A8], ids=lambda s: s.name)
def test_quant_act_matches_oracle_bit_for_bit(shape):
    say(f"[moe_quant_act] {shape.name}")
    x, _, _ = synth.make_gate_inputs(shape, device="cuda")
    cfg = B.config_of(shape)
    r = B.make_routing(cfg, shape.T)
    B.moe_quant_act(cfg, shape.T, x, r)
    torch.cuda.synchronize()
    codes, scales = w8a8.quant_1x128(to_f64(x).astype(np.float32))
    assert np.array_equal(r.act_q.cpu().numpy(), codes)
    assert np.array_equal(r.act_s.cpu().numpy().view(np.uint32), scales.view(np.uint32))


def _check(layer, tokens=None):
    shape = layer.shape
    mod = B.MoELayer(layer)
    T, K = shape.T, shape.top_k
    idx = torch.empty(T, K, dtype=torch.int32, device="cuda")
    w = torch.empty(T, K, dtype=torch.float32, device="cuda")
    out = mod.forward(layer.x, topk_idx=idx, topk_w=w)
    torch.cuda.synchronize()
    ref, _ = run_oracle(layer, tokens=tokens, force_idx=idx.cpu().numpy().astype(np.int64))
    got, u = to_f64(out), to_f64(layer.x)
    if tokens is not None:
        got, u = got[tokens], u[tokens]
    e_out, e_ffn = rel_err(got, ref), rel_err(got - u, ref - u)
    say(f"  rel err h'={e_out:.3g}  h'-u={e_ffn:.3g}  tol={TOL['fp8']}")
    assert np.all(np.isfinite(got))
    assert e_out <= TOL["fp8"] and e_ffn <= TOL["fp8"]
    return out, idx, w


@pytest.mark.parametrize("name", list(SHAPES))
def test_w8a8_forward_parity(name):
    _check(_layer(SHAPES[name]))


def test_w8a8_v3_prefill_sampled():
    shape = configs.V3_PREFILL_W8A8
    rng = np.random.default_rng(shape.seed + 100)
    toks = np.sort(rng.choice(shape.T, size=8, replace=False))
    toks[-1] = shape.T - 1
    _check(_layer(shape), tokens=toks)


def test_w8a8_steps_equal_forward():
    """gate -> permute -> quant_act -> expert_ffn -> combine == moe_forward, bit for bit."""
    layer = _layer(SHAPES["w8a8_ragged_2shared"])
    shape = layer.shape
    out2, idx2, w2 = _check(layer)
    cfg = B.config_of(shape)
    x = layer.x
    T, E, K, D, I = shape.T, shape.n_routed, shape.top_k, shape.dim, shape.inter_dim
    SI = shape.n_shared * I
    logits = torch.empty(T, E, dtype=torch.float32, device="cuda")
    idx = torch.empty(T, K, dtype=torch.int32, device="cuda")
    w = torch.empty(T, K, dtype=torch.float32, device="cuda")
    B.moe_gate(cfg, T, x, layer.w_gate, layer.bias, logits, idx, w)
    r = B.make_routing(cfg, T)
    B.moe_permute(cfg, T, idx, r)
    B.moe_quant_act(cfg, T, x, r)
    h = torch.empty(r.struct.max_rows, I, dtype=torch.bfloat16, device="cuda")
    y = torch.empty(r.struct.max_rows, D, dtype=torch.bfloat16, device="cuda")
    hs = torch.empty(T, SI, dtype=torch.bfloat16, device="cuda")
    z = torch.empty(T, D, dtype=torch.bfloat16, device="cuda")
    B.moe_expert_up(cfg, T, x, r, B.weights_of(layer), h, hs)
    B.moe_expert_down(cfg, T, r, B.weights_of(layer), h, hs, y, z)
    out = torch.empty_like(x)
    B.moe_combine(cfg, T, x, z, y, r, w, out)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2) and torch.equal(w, w2)
    assert torch.equal(out, out2)
