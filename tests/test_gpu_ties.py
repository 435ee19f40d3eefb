"""GPU parity with exact ties in the gate.

The pages leave ties open; the reading is that equal keys rank the lower expert
index first, and equal group scores the lower group index.  Ties only arise
from constructed inputs: here gate rows (and bias entries) are copied so that
whole triples of experts, and whole triples of groups, have bitwise-equal
logits.  Sorted keys then come in runs of three or four, so the top-k boundary (and the
topk_groups boundary) splits a run of equal values on most tokens.

For every token the GPU's experts must equal the oracle's selection replayed on
the GPU's own fp32 keys (a stable sort: lower index first on ties), and, where
the float64 keys certify the choice apart from the constructed ties, the
oracle's own float64 selection.  The tests also count the tokens on which a tie
straddles a boundary, so that they cannot pass without exercising the rule.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle_bridge import spec_of, to_f64
from parity import run_gate, say
from routed_expert_moe_amd import synth
from routed_expert_moe_amd.configs import LayerShape

pytestmark = pytest.mark.gpu


def _rep(E: int, G: int, K: int) -> np.ndarray:
    """Expert e copies the gate row of rep[e]: groups in triples, and inside a group experts in
    runs of 3 (of 4 when K is a multiple of 3), so that the K-th key ends inside a run."""
    gsz = E // G
    run = 3 if K % 3 else 4
    rep = np.empty(E, dtype=np.int64)
    for e in range(E):
        g, j = divmod(e, gsz)
        rep[e] = (g // 3 * 3) * gsz + (j // run * run)
    return rep


def _tied_layer(shape: LayerShape):
    x, wg, bias = synth.make_gate_inputs(shape, device="cpu")
    rep = torch.from_numpy(_rep(shape.n_routed, shape.n_groups, shape.top_k))
    wg = wg[rep].contiguous()
    if bias is not None:
        bias = bias[rep].contiguous()
    return x.cuda(), wg.cuda(), None if bias is None else bias.cuda()


class _Gate:
    def __init__(self, shape, x, w_gate, bias):
        self.shape, self.x, self.w_gate, self.bias = shape, x, w_gate, bias


def _boundary_ties(key: np.ndarray, spec, has_bias: bool):
    """Tokens whose K-th and (K+1)-th surviving keys are equal, and whose topk_groups-th
    and next group scores are equal (evaluated on the given keys)."""
    T, E = key.shape
    masked = key
    group_tie = np.zeros(T, dtype=bool)
    if spec.n_groups > 1:
        gs = oracle.group_scores(key, spec.n_groups, top2=has_bias)
        srt = -np.sort(-gs, axis=-1)
        if spec.topk_groups < spec.n_groups:
            group_tie = srt[:, spec.topk_groups - 1] == srt[:, spec.topk_groups]
        keep = np.argsort(-gs, axis=-1, kind="stable")[:, : spec.topk_groups]
        on = np.zeros((T, spec.n_groups), dtype=bool)
        np.put_along_axis(on, keep, True, axis=-1)
        masked = np.where(np.repeat(on, E // spec.n_groups, axis=1), key, -np.inf)
    srt = -np.sort(-masked, axis=-1)
    expert_tie = srt[:, spec.top_k - 1] == srt[:, spec.top_k] if spec.top_k < E else np.zeros(T, bool)
    return expert_tie, group_tie


def _run_case(shape: LayerShape):
    say(f"[ties] {shape.name} T={shape.T} E={shape.n_routed} G={shape.n_groups} "
        f"TG={shape.topk_groups} K={shape.top_k} {shape.score}")
    x, wg, bias = _tied_layer(shape)
    gate = _Gate(shape, x, wg, bias)
    logits, keys, idx, w = run_gate(gate)
    rep = _rep(shape.n_routed, shape.n_groups, shape.top_k)
    # the construction: copied gate rows give bitwise-equal logits and keys on the GPU
    assert np.array_equal(logits, logits[:, rep]), "copied gate rows gave different logits"
    assert np.array_equal(keys, keys[:, rep]), "copied gate rows gave different keys"
    spec = spec_of(shape)
    has_bias = bias is not None
    # (1) every token: the GPU's experts are the lower-index-first selection on its own keys
    replay = oracle.select_experts(keys.astype(np.float32), spec, has_bias)
    bad = np.nonzero((replay != idx).any(axis=1))[0]
    assert bad.size == 0, f"tokens {bad[:10]}: GPU {idx[bad[:3]]} vs replay {replay[bad[:3]]}"
    e_tie, g_tie = _boundary_ties(keys.astype(np.float32), spec, has_bias)
    say(f"  tokens with an expert tie at the top-k boundary: {int(e_tie.sum())}/{shape.T}, "
        f"with a group tie at the topk_groups boundary: {int(g_tie.sum())}/{shape.T}")
    assert e_tie.sum() > shape.T // 4
    if shape.n_groups > 1 and shape.topk_groups < shape.n_groups:
        assert g_tie.sum() > shape.T // 4
    # (2) the float64 oracle: the same copies tie exactly in float64 too; its selection must
    # equal the GPU's on every token whose remaining (non-constructed) gaps exceed 4 eps
    g = oracle.gate(to_f64(x), to_f64(wg), None if bias is None else bias.cpu().numpy().astype(np.float64), spec)
    eps = float(np.max(np.abs(keys.astype(np.float64) - g.key)))
    # distinct key values per token: the gaps between different runs of equal keys
    uniq_gap = np.array([np.min(np.diff(np.unique(row))) if np.unique(row).size > 1 else np.inf
                         for row in g.key])
    gs = oracle.group_scores(g.key, shape.n_groups, top2=has_bias) if shape.n_groups > 1 else None
    grp_gap = (np.array([np.min(np.diff(np.unique(row))) if np.unique(row).size > 1 else np.inf for row in gs])
               if gs is not None else np.full(shape.T, np.inf))
    cert = (uniq_gap > 4 * eps) & (grp_gap > 8 * eps)
    mism = np.nonzero(cert & (idx != g.idx).any(axis=1))[0]
    say(f"  eps={eps:.3g}, certified {int(cert.sum())}/{shape.T}")
    assert mism.size == 0, f"certified tokens {mism[:10]} differ from the float64 oracle"
    assert cert.mean() > 0.5
    # (3) the weights follow the chosen experts (equal scores give equal weights)
    assert (np.diff(idx, axis=1) > 0).all()


CASES = {
    # the tiny layer's group shape (16 experts, 4 groups keep 2, top-4), fp32 SIMT logits
    "tiny_groups_f32": LayerShape(
        name="ties_tiny_f32", T=200, dim=256, n_routed=16, n_groups=4, topk_groups=2, top_k=4,
        n_shared=1, inter_dim=128, score="sigmoid", route_scale=2.5, act="f32", weight="f32",
        seed=51, bias_range=0.1),
    # the V3 group shape (256 experts, 8 groups keep 4, top-8): bf16 GEMV logits (T < 64)
    "v3_groups_gemv": LayerShape(
        name="ties_v3_gemv", T=40, dim=7168, n_routed=256, n_groups=8, topk_groups=4, top_k=8,
        n_shared=1, inter_dim=2048, score="sigmoid", route_scale=2.5, act="bf16", weight="bf16",
        seed=52, bias_range=0.05),
    # ... and MFMA logits (T >= 64)
    "v3_groups_mfma": LayerShape(
        name="ties_v3_mfma", T=600, dim=7168, n_routed=256, n_groups=8, topk_groups=4, top_k=8,
        n_shared=1, inter_dim=2048, score="sigmoid", route_scale=2.5, act="bf16", weight="bf16",
        seed=53, bias_range=0.05),
    # the V3 group shape without a bias: group score = max key
    "v3_groups_nobias": LayerShape(
        name="ties_v3_nobias", T=300, dim=512, n_routed=256, n_groups=8, topk_groups=4, top_k=8,
        n_shared=1, inter_dim=256, score="sigmoid", route_scale=2.5, act="bf16", weight="bf16",
        seed=54),
    # softmax scoring (V2-style, no groups), GEMV and MFMA logits
    "softmax_gemv": LayerShape(
        name="ties_softmax_gemv", T=33, dim=2048, n_routed=64, n_groups=1, topk_groups=1, top_k=6,
        n_shared=2, inter_dim=1408, score="softmax", route_scale=1.0, act="bf16", weight="bf16",
        seed=55),
    "softmax_mfma": LayerShape(
        name="ties_softmax_mfma", T=512, dim=2048, n_routed=64, n_groups=1, topk_groups=1, top_k=6,
        n_shared=2, inter_dim=1408, score="softmax", route_scale=1.0, act="bf16", weight="bf16",
        seed=56),
}


@pytest.mark.parametrize("name", list(CASES))
def test_exact_ties_lowest_index(name):
    _run_case(CASES[name])
