"""GPU parity of the layer backward (moe_backward) against the float64 oracle.

The forward runs on the GPU through the step entry points; its routing (the
GPU's selection) is handed to the oracle as force_idx, so both sides
differentiate the same piecewise-smooth function.  Every gradient is compared
as max|err| / max|ref| <= 2e-2 (the bf16 bound of the forward outputs: the
backward rounds dy, h, da/dc and dlogits to bf16 once each as GEMM operands,
relative 2^-9, and accumulates in fp32).  Experts no token chose must get
exactly zero gradients, and two calls must agree bit for bit.
"""
import numpy as np
import pytest
import torch

from oracle import backward as obw
from oracle_bridge import bias_f64, expert_fn, shared_pair, spec_of, to_f64
from parity import rel_err, say
from routed_expert_moe_amd import binding as B
from routed_expert_moe_amd import synth
from routed_expert_moe_amd.configs import LayerShape

pytestmark = pytest.mark.gpu

TOL = 2e-2

SHAPES = {
    # 24 rows per expert on average: the 16-row streaming recompute path
    "skinny_groups_bias": LayerShape(
        name="bwd_skinny", T=96, dim=256, n_routed=16, n_groups=4, topk_groups=2, top_k=4,
        n_shared=1, inter_dim=128, score="sigmoid", route_scale=2.5, act="bf16", weight="bf16",
        seed=31, bias_range=0.1),
    # 128 rows per expert: the MFMA recompute path, two shared experts, softmax
    "mfma_softmax": LayerShape(
        name="bwd_mfma", T=512, dim=512, n_routed=16, n_groups=1, topk_groups=1, top_k=4,
        n_shared=2, inter_dim=256, score="softmax", route_scale=1.0, act="bf16", weight="bf16", seed=32),
    # ragged: inter 136 (no multiple of 128), 24 experts, no shared expert, no residual
    "ragged_noshared": LayerShape(
        name="bwd_ragged", T=200, dim=384, n_routed=24, n_groups=1, topk_groups=1, top_k=6,
        n_shared=0, inter_dim=136, score="sigmoid", route_scale=1.5, act="bf16", weight="bf16",
        seed=33, add_residual=0),
    # one token: K of the E experts get one row each (16-row tiles), the rest nothing
    "single_token": LayerShape(
        name="bwd_t1", T=1, dim=256, n_routed=16, n_groups=4, topk_groups=2, top_k=4,
        n_shared=1, inter_dim=128, score="sigmoid", route_scale=2.5, act="bf16", weight="bf16",
        seed=35, bias_range=0.1),
    # ragged T (37): partial dense tiles for the shared expert and the gate
    "ragged_T37_softmax_norm": LayerShape(
        name="bwd_t37", T=37, dim=384, n_routed=32, n_groups=1, topk_groups=1, top_k=3,
        n_shared=2, inter_dim=64, score="softmax", route_scale=1.0, norm_topk=1, act="bf16",
        weight="bf16", seed=36),
    # Zipf-skewed gate: several experts get no token and must get zero gradients
    "skewed_idle_experts": LayerShape(
        name="bwd_skewed", T=64, dim=256, n_routed=32, n_groups=1, topk_groups=1, top_k=2,
        n_shared=1, inter_dim=128, score="sigmoid", route_scale=2.5, act="bf16", weight="bf16",
        seed=34, zipf=2.0),
}


def _forward(layer):
    s = layer.shape
    cfg = B.config_of(s)
    T, E, K, D, I, S = s.T, s.n_routed, s.top_k, s.dim, s.inter_dim, s.n_shared
    dev = layer.x.device
    logits = torch.empty(T, E, dtype=torch.float32, device=dev)
    idx = torch.empty(T, K, dtype=torch.int32, device=dev)
    w = torch.empty(T, K, dtype=torch.float32, device=dev)
    B.moe_gate(cfg, T, layer.x, layer.w_gate, layer.bias, logits, idx, w)
    r = B.make_routing(cfg, T)
    B.moe_permute(cfg, T, idx, r)
    R = r.struct.max_rows
    h = torch.empty(R, I, dtype=torch.bfloat16, device=dev)
    y = torch.empty(R, D, dtype=torch.bfloat16, device=dev)
    hs = torch.empty(T, S * I, dtype=torch.bfloat16, device=dev) if S else None
    z = torch.empty(T, D, dtype=torch.bfloat16, device=dev) if S else None
    wts = B.weights_of(layer)
    B.moe_expert_ffn(cfg, T, layer.x, r, wts, h, y, hs, z)
    return cfg, wts, logits, idx, w, r, y


def _backward(layer, cfg, wts, logits, idx, w, r, y, dout):
    g = B.Grads.empty(cfg, layer.shape.T, torch.bfloat16)
    B.moe_backward(cfg, layer.shape.T, layer.x, wts, r, idx, w, logits, y, dout, g)
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("name", list(SHAPES))
def test_backward_matches_oracle(name):
    s = SHAPES[name]
    say(f"[moe_backward] {name} T={s.T} D={s.dim} E={s.n_routed} K={s.top_k} I={s.inter_dim} S={s.n_shared}")
    layer = synth.make_layer(s, device="cuda")
    dout = synth.make_dout(s, device="cuda")
    fwd = _forward(layer)
    g = _backward(layer, *fwd, dout)
    idx = fwd[3].cpu().numpy().astype(np.int64)

    ref = obw.moe_layer_backward(to_f64(layer.x), to_f64(layer.w_gate), bias_f64(layer), expert_fn(layer),
                                 shared_pair(layer), spec_of(s), to_f64(dout), force_idx=idx)
    errs = {"dx": rel_err(to_f64(g.dx), ref.dx), "dw_gate": rel_err(g.dw_gate.cpu().numpy(), ref.dw_gate)}
    dw13, dw2 = g.dw13.cpu().numpy(), g.dw2.cpu().numpy()
    chosen = set(int(e) for e in np.unique(idx))
    for e in range(s.n_routed):
        if e in chosen:
            errs[f"dw13[{e}]"] = rel_err(dw13[e], ref.dw13[e])
            errs[f"dw2[{e}]"] = rel_err(dw2[e], ref.dw2[e])
        else:
            assert not dw13[e].any() and not dw2[e].any(), f"expert {e} has no tokens but non-zero gradients"
    if s.n_shared:
        errs["dsw13"] = rel_err(g.dsw13.cpu().numpy(), ref.dsw13)
        errs["dsw2"] = rel_err(g.dsw2.cpu().numpy(), ref.dsw2)
    if name == "skewed_idle_experts":
        assert len(chosen) < s.n_routed, "the skewed case should leave experts idle"
    worst = max(errs, key=errs.get)
    say(f"  worst {worst} {errs[worst]:.3g}; dx {errs['dx']:.3g} dw_gate {errs['dw_gate']:.3g}")
    bad = {k: v for k, v in errs.items() if not v <= TOL}
    assert not bad, bad

    # the same call again: bitwise identical
    g2 = _backward(layer, *fwd, dout)
    for a, b in ((g.dx, g2.dx), (g.dw_gate, g2.dw_gate), (g.dw13, g2.dw13), (g.dw2, g2.dw2)):
        assert torch.equal(a, b)


def test_backward_rejects_unsupported_and_small_workspace():
    s = SHAPES["skinny_groups_bias"]
    cfg = B.config_of(s)
    need = B.moe_backward_workspace_size(cfg, s.T)
    layer = synth.make_layer(s, device="cuda")
    fwd = _forward(layer)
    dout = synth.make_dout(s, device="cuda")
    g = B.Grads.empty(cfg, s.T, torch.bfloat16)
    small = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(B.MoeError) as ei:
        B.moe_backward(cfg, s.T, layer.x, fwd[1], fwd[5], fwd[3], fwd[4], fwd[2], fwd[6], dout, g, workspace=small)
    assert ei.value.status == B.MOE_ERR_WORKSPACE
    f32 = B.config_of(s.with_(act="f32", weight="f32"))
    with pytest.raises(B.MoeError) as ei:
        B.moe_backward_workspace_size(f32, s.T)
    assert ei.value.status == B.MOE_ERR_UNSUPPORTED


def test_backward_v3_prefill_sampled():
    """The V3 prefill layer at its full size (T=8192, the batch bench.py times), against
    the oracle computed for just the sampled outputs, each of which depends on a known
    part of the batch only:
      * dx of a token sample (a token's dx involves its own gate row, experts and dout);
      * dW13 / dW2 of the least and the most loaded expert (the rows it received);
      * rows e of dW_gate for those experts (with sigmoid scores a token's gate gradient
        is zero outside its chosen experts, so row e sums over the tokens that chose e);
      * a seeded slice of 64 hidden units of the shared expert's dW13 (their W1 and W3
        rows) and dW2 (their columns): SwiGLU hidden units do not interact, so the
        gradient of the sliced FFN is the slice of the full gradient."""
    import oracle
    from routed_expert_moe_amd import configs
    s = configs.V3_PREFILL_BF16
    say("[moe_backward] v3 prefill T=8192, sampled")
    layer = synth.make_layer(s, device="cuda")
    dout = synth.make_dout(s, device="cuda")
    fwd = _forward(layer)
    g = _backward(layer, *fwd, dout)
    idx = fwd[3].cpu().numpy().astype(np.int64)
    spec = spec_of(s)
    x64 = to_f64(layer.x)
    wg64 = to_f64(layer.w_gate)
    d64 = to_f64(dout)
    get = expert_fn(layer, fast=True)
    sh = shared_pair(layer)

    # dx of sampled tokens: the oracle's backward restricted to those tokens is
    # exact, since dx_t only involves token t's gate row, experts and dout_t
    rng = np.random.default_rng(2024)
    toks = np.sort(rng.choice(s.T, 48, replace=False))
    toks[-1] = s.T - 1
    want = obw.moe_layer_backward(x64[toks], wg64, bias_f64(layer), get, sh, spec, d64[toks],
                                  force_idx=idx[toks]).dx
    err = rel_err(to_f64(g.dx)[toks], want)
    say(f"  dx ({toks.size} tokens) {err:.3g}")
    assert err <= TOL

    counts = np.bincount(idx.ravel(), minlength=s.n_routed)
    least = int(np.argmin(np.where(counts > 0, counts, 1 << 30)))
    busiest = int(np.argmax(counts))
    gt = oracle.gate(x64, wg64, bias_f64(layer), spec, force_idx=idx)
    dwg = g.dw_gate.cpu().numpy()
    for e in (least, busiest):
        # the expert's weight gradients from every row it received
        rows, slot = np.nonzero(idx == e)
        w13, w2 = get(e)
        dy = gt.w[rows, slot][:, None] * d64[rows]
        _, dw13, dw2 = obw.swiglu_ffn_backward(x64[rows], w13, w2, dy)
        e13 = rel_err(g.dw13[e].cpu().numpy(), dw13)
        e2 = rel_err(g.dw2[e].cpu().numpy(), dw2)
        # row e of dW_gate: the backward of the tokens that chose e
        ref = obw.moe_layer_backward(x64[rows], wg64, bias_f64(layer), get, sh, spec, d64[rows],
                                     force_idx=idx[rows])
        eg = rel_err(dwg[e], ref.dw_gate[e])
        say(f"  expert {e} ({rows.size} rows): dw13 {e13:.3g} dw2 {e2:.3g} dw_gate[e] {eg:.3g}")
        assert e13 <= TOL and e2 <= TOL and eg <= TOL

    # the shared expert on a slice of its hidden units, over all tokens (dz = dout)
    SI = s.n_shared * s.inter_dim
    J = np.sort(rng.choice(SI, 64, replace=False))
    sw13, sw2 = sh
    _, d13, d2 = obw.swiglu_ffn_backward(x64, sw13[np.concatenate([J, SI + J])], sw2[:, J], d64)
    e13 = rel_err(g.dsw13.cpu().numpy()[np.concatenate([J, SI + J])], d13)
    e2 = rel_err(g.dsw2.cpu().numpy()[:, J], d2)
    say(f"  shared expert, 64 hidden units: dsw13 {e13:.3g} dsw2 {e2:.3g}")
    assert e13 <= TOL and e2 <= TOL
