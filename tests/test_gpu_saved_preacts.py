"""GPU: the training forward that keeps the SwiGLU inputs (moe_expert_ffn_save) and the
backward that reads them instead of recomputing (moe_backward_saved).

The SwiGLU experts of the DeepSeek-V3 notes page compute a = W1_e x and c = W3_e x and
feed silu(a) * c to W2_e; the layer backward needs a and c again.  Checked here:
  * the forward outputs (h, y_pairs, hs, z) equal moe_expert_ffn's bit for bit on every
    real row, so keeping a and c changes nothing else;
  * every real row of ab (and every token of abs) against the oracle's a and c
    (oracle.swiglu_preacts, float64), within fp32 accumulation error of the bf16 sums;
  * moe_backward_saved gives the same gradients as moe_backward bit for bit, on the
    backward test shapes (the 16-row streaming path, where the save falls back to one
    more fp32 GEMM, and the 128-row prefill path, where the expert GEMM writes a and c
    from its accumulators), a 128-row shape whose K rules out the prefill expert GEMM
    (the fallback again), V2-Lite and the V3 prefill batch at full size."""
import numpy as np
import pytest
import torch

import oracle
from oracle_bridge import expert_fn, shared_pair, to_f64
from parity import say
from routed_expert_moe_amd import binding as B
from routed_expert_moe_amd import configs, synth
from routed_expert_moe_amd.configs import LayerShape
from test_gpu_backward import SHAPES as BWD_SHAPES

pytestmark = pytest.mark.gpu

# |a_gpu - a| <= PRE_TOL * sum_j |x_j W_ij|: fp32 sums of exact bf16 products
PRE_TOL = 1e-4


def _ffn(layer, save: bool):
    """gate -> permute -> expert FFN (with or without the saved pre-activations)."""
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
    out = {"h": torch.empty(R, I, dtype=torch.bfloat16, device=dev),
           "y": torch.empty(R, D, dtype=torch.bfloat16, device=dev),
           "hs": torch.empty(T, S * I, dtype=torch.bfloat16, device=dev) if S else None,
           "z": torch.empty(T, D, dtype=torch.bfloat16, device=dev) if S else None}
    wts = B.weights_of(layer)
    if save:
        out["ab"] = torch.empty(R, 2 * I, dtype=torch.float32, device=dev)
        out["abs"] = torch.empty(T, 2 * S * I, dtype=torch.float32, device=dev) if S else None
        B.moe_expert_ffn_save(cfg, T, layer.x, r, wts, out["h"], out["y"], out["hs"], out["z"],
                              out["ab"], out["abs"])
    else:
        B.moe_expert_ffn(cfg, T, layer.x, r, wts, out["h"], out["y"], out["hs"], out["z"])
    torch.cuda.synchronize()
    return cfg, wts, logits, idx, w, r, out


def _used(r):
    """The routed rows in use (tiles times tile rows); the buffers' tails are unset."""
    return int(r.n_tiles.item()) * r.struct.tile_m


def _grads(layer, cfg, wts, logits, idx, w, r, out, dout, saved=None):
    g = B.Grads.empty(cfg, layer.shape.T, torch.bfloat16)
    if saved is None:
        B.moe_backward(cfg, layer.shape.T, layer.x, wts, r, idx, w, logits, out["y"], dout, g)
    else:
        B.moe_backward_saved(cfg, layer.shape.T, layer.x, wts, r, idx, w, logits, out["y"], dout,
                             saved["ab"], saved["abs"], g)
    torch.cuda.synchronize()
    return g


def _check_preacts(layer, idx, r, ab, abs_, experts=None, tokens=None):
    """ab's real rows (every row, or up to 16 rows of each of the given experts) and abs
    (every token, or the given ones) against the oracle's a and c."""
    s = layer.shape
    K, I, S = s.top_k, s.inter_dim, s.n_shared
    x64 = to_f64(layer.x)
    sp = r.sorted_pair[:_used(r)].cpu().numpy()
    idx_np = idx.cpu().numpy()
    real = np.nonzero(sp >= 0)[0]
    if experts is None:
        rows = real
    else:
        row_e = idx_np.ravel()[sp[real]]
        rows = np.concatenate([real[row_e == e][:8] for e in experts] +
                              [real[row_e == e][-8:] for e in experts])
        rows = np.unique(rows)
    get = expert_fn(layer, fast=True)
    ab_np = ab[torch.as_tensor(rows, device=ab.device)].cpu().numpy().astype(np.float64)
    worst = 0.0
    by_expert = {}
    for q, row in enumerate(rows):
        t, slot = divmod(int(sp[row]), K)
        by_expert.setdefault(int(idx_np[t, slot]), []).append((q, t))
    for e, lst in by_expert.items():
        w13, _ = get(e)
        qs = np.array([q for q, _ in lst])
        ts = np.array([t for _, t in lst])
        a, c = oracle.swiglu_preacts(x64[ts], w13)
        scale = np.abs(x64[ts]) @ np.abs(w13).T
        err = np.abs(ab_np[qs] - np.concatenate([a, c], axis=1)) / np.maximum(scale, 1e-300)
        worst = max(worst, float(err.max()))
    say(f"  ab: {len(rows)} rows of {real.size}, worst error {worst:.3g} of the sum of |terms|")
    assert worst <= PRE_TOL
    if S:
        sw13, _ = shared_pair(layer)
        toks = np.arange(s.T) if tokens is None else np.asarray(tokens)
        a, c = oracle.swiglu_preacts(x64[toks], sw13)
        got = abs_[torch.as_tensor(toks, device=abs_.device)].cpu().numpy().astype(np.float64)
        scale = np.abs(x64[toks]) @ np.abs(sw13).T
        err = float((np.abs(got - np.concatenate([a, c], axis=1)) / np.maximum(scale, 1e-300)).max())
        say(f"  abs: {toks.size} tokens, worst error {err:.3g} of the sum of |terms|")
        assert err <= PRE_TOL


def _same_forward(r, a, b):
    real = torch.nonzero(r.sorted_pair[:_used(r)] >= 0).flatten()
    for k in ("h", "y"):
        assert torch.equal(a[k][real], b[k][real]), k
    for k in ("hs", "z"):
        if a[k] is not None:
            assert torch.equal(a[k], b[k]), k


def _same_grads(g1, g2, shared):
    names = ["dx", "dw_gate", "dw13", "dw2"] + (["dsw13", "dsw2"] if shared else [])
    for n in names:
        assert torch.equal(getattr(g1, n), getattr(g2, n)), n


CASES = dict(BWD_SHAPES)
CASES["v2lite_bf16_T512"] = configs.V2_LITE_BF16
# dim 352 (not a multiple of 64): the 128-row MFMA path without the prefill expert GEMM,
# so the save falls back to the separate fp32 GEMM there too
CASES["mfma_dim352"] = LayerShape(
    name="save_d352", T=512, dim=352, n_routed=16, n_groups=4, topk_groups=2, top_k=4, n_shared=1,
    inter_dim=128, score="sigmoid", route_scale=2.5, act="bf16", weight="bf16", seed=38, bias_range=0.1)


@pytest.mark.parametrize("name", list(CASES))
def test_saved_preacts_match_forward_oracle_and_backward(name):
    s = CASES[name]
    say(f"[moe_expert_ffn_save / moe_backward_saved] {name} T={s.T} D={s.dim} E={s.n_routed} "
        f"K={s.top_k} I={s.inter_dim} S={s.n_shared}")
    layer = synth.make_layer(s, device="cuda")
    dout = synth.make_dout(s, device="cuda")
    cfg, wts, logits, idx, w, r, plain = _ffn(layer, save=False)
    _, _, _, _, _, r2, saved = _ffn(layer, save=True)
    assert _used(r) == _used(r2) and torch.equal(r.sorted_pair[:_used(r)], r2.sorted_pair[:_used(r)])
    _same_forward(r, plain, saved)
    _check_preacts(layer, idx, r, saved["ab"], saved["abs"])
    g1 = _grads(layer, cfg, wts, logits, idx, w, r, plain, dout)
    g2 = _grads(layer, cfg, wts, logits, idx, w, r2, saved, dout, saved=saved)
    _same_grads(g1, g2, s.n_shared > 0)


def test_saved_preacts_v3_prefill_full_size():
    """The V3 prefill batch (T=8192, 256-row expert chunks and 128-row ones, the shared
    expert as a dense segment): forward outputs and gradients bitwise equal, a and c of a
    seeded sample of rows (every column) against the oracle."""
    s = configs.V3_PREFILL_BF16
    say("[moe_expert_ffn_save / moe_backward_saved] v3 prefill T=8192")
    layer = synth.make_layer(s, device="cuda")
    dout = synth.make_dout(s, device="cuda")
    cfg, wts, logits, idx, w, r, plain = _ffn(layer, save=False)
    g1 = _grads(layer, cfg, wts, logits, idx, w, r, plain, dout)
    _, _, _, _, _, r2, saved = _ffn(layer, save=True)
    assert _used(r) == _used(r2) and torch.equal(r.sorted_pair[:_used(r)], r2.sorted_pair[:_used(r)])
    _same_forward(r, plain, saved)
    counts = np.bincount(idx.cpu().numpy().ravel(), minlength=s.n_routed)
    rng = np.random.default_rng(77)
    experts = [int(np.argmax(counts)), int(np.argmin(np.where(counts > 0, counts, 1 << 30)))] + \
        [int(e) for e in rng.choice(s.n_routed, 4, replace=False)]
    tokens = np.unique(np.concatenate([[0, s.T - 1], rng.choice(s.T, 62, replace=False)]))
    _check_preacts(layer, idx, r, saved["ab"], saved["abs"], experts=experts, tokens=tokens)
    del plain
    g2 = _grads(layer, cfg, wts, logits, idx, w, r2, saved, dout, saved=saved)
    _same_grads(g1, g2, True)
