"""Pins for the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: hand-worked
examples (tests/golden), closed forms, brute-force definitions on tiny inputs,
invariants the pages state, and library decoders.  A plausible slip in the
oracle (a dropped term, a wrong sign, a swapped or transposed operand, the
wrong group score, bias leaking into the weights) fails at least one of them.
"""
import itertools
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import Spec

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _fixture(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            k, v = (s.strip() for s in line.split("=", 1))
            vals[k] = v
    return vals


def _floats(s):
    return [float(t) for t in s.split()]


def _matrix(s):
    return np.array([_floats(r) for r in s.split(";")], dtype=np.float64)


# ---------------------------------------------------------------- decoders
def test_decode_e4m3_all_codes_match_library():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.decode_e4m3(codes)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(lib))
    ok = ~np.isnan(lib)
    assert np.array_equal(ours[ok], lib[ok])


def test_decode_e4m3_format_points():
    # OCP e4m3fn: 0x7E = 448 (max), 0x08 = 2^-6 (min normal), 0x01 = 2^-9 (min subnormal)
    pts = {0x00: 0.0, 0x38: 1.0, 0xB8: -1.0, 0x7E: 448.0, 0xFE: -448.0, 0x08: 2.0 ** -6,
           0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x3C: 1.5, 0x40: 2.0}
    for c, v in pts.items():
        assert oracle.decode_e4m3(np.array([c], np.uint8))[0] == v, hex(c)
    assert np.isnan(oracle.decode_e4m3(np.array([0x7F, 0xFF], np.uint8))).all()


def test_decode_bf16_all_patterns_match_library():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.decode_bf16(bits)
    lib = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(lib))
    ok = ~np.isnan(lib)
    assert np.array_equal(ours[ok], lib[ok])


def test_dequant_block128_scales_each_block():
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 256, size=(256, 384), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x12     # no NaN codes
    scales = rng.uniform(0.01, 2.0, size=(2, 3)).astype(np.float32)
    got = oracle.dequant_e4m3_block128(codes, scales)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for bi in range(2):
        for bj in range(3):
            blk = (slice(128 * bi, 128 * bi + 128), slice(128 * bj, 128 * bj + 128))
            assert np.array_equal(got[blk], lib[blk] * np.float64(scales[bi, bj]))


# ---------------------------------------------------------------- gate, brute force
def test_gate_logits_brute_force():
    rng = np.random.default_rng(1)
    x, w = rng.normal(size=(3, 7)), rng.normal(size=(5, 7))
    got = oracle.gate_logits(x, w)
    for t in range(3):
        for e in range(5):
            assert abs(got[t, e] - math.fsum(x[t, j] * w[e, j] for j in range(7))) < 1e-14


def test_scores_brute_force():
    rng = np.random.default_rng(2)
    l = rng.normal(size=(4, 6)) * 3
    b = rng.uniform(-0.1, 0.1, size=6)
    s, key = oracle.gate_scores(l, "sigmoid", b)
    for t in range(4):
        for e in range(6):
            sig = 1.0 / (1.0 + math.exp(-l[t, e]))
            assert abs(s[t, e] - sig) < 1e-15
            assert abs(key[t, e] - (sig + b[e])) < 1e-15
    p, key = oracle.gate_scores(l, "softmax", None)
    for t in range(4):
        den = math.fsum(math.exp(v) for v in l[t])
        for e in range(6):
            assert abs(p[t, e] - math.exp(l[t, e]) / den) < 1e-15
    assert np.array_equal(key, l)      # ranking by logit = ranking by probability


def _brute_select(key, E, G, TG, K, top2):
    """Definition: an item is kept iff fewer than the allowed number beat it
    under (value descending, index ascending).  Group score by exhaustive pairs."""
    size = E // G
    keep_groups = list(range(G))
    if G > 1:
        gs = []
        for j in range(G):
            vals = [key[j * size + i] for i in range(size)]
            if top2:
                gs.append(max(vals[a] + vals[b] for a in range(size) for b in range(size) if a != b))
            else:
                gs.append(max(vals))
        keep_groups = [j for j in range(G)
                       if sum(1 for i in range(G) if gs[i] > gs[j] or (gs[i] == gs[j] and i < j)) < TG]
    alive = [e for e in range(E) if e // size in keep_groups]
    chosen = [e for e in alive
              if sum(1 for f in alive if key[f] > key[e] or (key[f] == key[e] and f < e)) < K]
    return sorted(chosen)


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
@pytest.mark.parametrize("E,G,TG,K", [(16, 4, 2, 4), (16, 1, 1, 4), (12, 3, 2, 5), (8, 4, 4, 3),
                                      (16, 8, 3, 6), (6, 2, 1, 2), (32, 8, 4, 8)])
def test_select_matches_brute_force(dtype, E, G, TG, K):
    rng = np.random.default_rng(E * 131 + G * 17 + K)
    for trial in range(120):
        top2 = bool(trial % 2)
        if trial % 3 == 0:   # coarse grid -> many exact ties
            key = (rng.integers(-3, 4, size=(1, E)) / 4.0).astype(dtype)
        else:
            key = rng.normal(size=(1, E)).astype(dtype)
        spec = Spec(n_routed=E, n_groups=G, topk_groups=TG, top_k=K, score="sigmoid", route_scale=1.0)
        got = oracle.select_experts(key, spec, has_bias=top2)[0].tolist()
        assert got == _brute_select(key[0], E, G, TG, K, top2), (trial, key)


def test_select_exact_ties_take_lowest_index():
    key = np.zeros((1, 16))
    spec = Spec(n_routed=16, n_groups=4, topk_groups=2, top_k=4, score="sigmoid", route_scale=1.0)
    assert oracle.select_experts(key, spec, has_bias=True)[0].tolist() == [0, 1, 2, 3]
    spec1 = Spec(n_routed=16, n_groups=1, topk_groups=1, top_k=3, score="softmax", route_scale=1.0)
    assert oracle.select_experts(key, spec1, has_bias=False)[0].tolist() == [0, 1, 2]


def test_selection_margins_certify_perturbations():
    rng = np.random.default_rng(9)
    spec = Spec(n_routed=32, n_groups=8, topk_groups=4, top_k=8, score="sigmoid", route_scale=2.5)
    key = rng.normal(size=(400, 32))
    base = oracle.select_experts(key, spec, has_bias=True)
    eg, gg = oracle.selection_margins(key, spec, has_bias=True)
    # brute-force the gaps from sorted values
    gs = oracle.group_scores(key, 8, top2=True)
    srt = np.sort(gs, axis=1)[:, ::-1]
    assert np.allclose(gg, srt[:, 3] - srt[:, 4])
    for t in range(400):
        eps = 0.24 * min(eg[t], gg[t] / 2.0)
        pert = key[t:t + 1] + rng.uniform(-eps, eps, size=(1, 32))
        assert (oracle.select_experts(pert, spec, has_bias=True) == base[t]).all()
    # a perturbation of the size of the gap can flip the selection
    t = int(np.argmin(eg))
    assert eg[t] > 0


# ---------------------------------------------------------------- golden examples
def test_golden_group_limited_sigmoid_gate():
    g = _fixture("gate_worked_example.txt")
    E, G, TG, K = (int(g[k]) for k in ("n_routed", "n_groups", "topk_groups", "top_k"))
    s = np.array(_floats(g["scores"]))
    logits = np.log(s / (1.0 - s))
    x = np.zeros((1, E))
    x[0, 0] = 1.0
    w_gate = np.zeros((E, E))
    w_gate[:, 0] = logits
    spec = Spec(n_routed=E, n_groups=G, topk_groups=TG, top_k=K, score=g["score"],
                route_scale=float(g["route_scale"]))
    bias = np.array(_floats(g["bias"]))
    res = oracle.gate(x, w_gate, bias, spec)
    assert np.allclose(oracle.group_scores(res.key, G, top2=True)[0], _floats(g["expect_group_scores"]), atol=1e-12)
    assert res.idx[0].tolist() == [int(v) for v in g["expect_idx"].split()]
    assert np.allclose(res.w[0], _floats(g["expect_w"]), atol=1e-12)


def test_golden_softmax_gate():
    g = _fixture("softmax_worked_example.txt")
    E, K = int(g["n_routed"]), int(g["top_k"])
    p = np.array(_floats(g["probs"]))
    x = np.zeros((1, E))
    x[0, 0] = 1.0
    w_gate = np.zeros((E, E))
    w_gate[:, 0] = np.log(p)
    spec = Spec(n_routed=E, n_groups=1, topk_groups=1, top_k=K, score="softmax", route_scale=1.0)
    res = oracle.gate(x, w_gate, None, spec)
    assert res.idx[0].tolist() == [int(v) for v in g["expect_idx"].split()]
    assert np.allclose(res.w[0], _floats(g["expect_w"]), atol=1e-14)


def test_golden_layer_output():
    g = _fixture("layer_worked_example.txt")
    u = np.array([_floats(g["u"])])
    w_gate = _matrix(g["gate_rows"])
    w13_1, w2_1 = _matrix(g["expert1_w13"]), _matrix(g["expert1_w2"])
    experts = {0: (np.zeros_like(w13_1), np.zeros_like(w2_1)), 1: (w13_1, w2_1)}
    shared = (_matrix(g["shared_w13"]), _matrix(g["shared_w2"]))
    spec = Spec(n_routed=2, n_groups=1, topk_groups=1, top_k=1, score="sigmoid",
                route_scale=float(g["route_scale"]))
    out, res = oracle.moe_layer(u, w_gate, None, experts.__getitem__, shared, spec)
    assert res.idx[0].tolist() == [int(g["expect_idx"])]
    assert np.allclose(out[0], _floats(g["expect_out"]), rtol=0, atol=1e-13)


def test_page_config_constants():
    from routed_expert_moe_amd import configs
    g = _fixture("page_configs.txt")
    for c in (configs.V3_PREFILL_BF16, configs.V3_DECODE_FP8):
        assert c.dim == int(g["v3.dim"]) and c.n_routed == int(g["v3.n_routed"])
        assert c.n_shared == int(g["v3.n_shared"]) and c.top_k == int(g["v3.top_k"])
        assert c.n_groups == int(g["v3.n_groups"]) and c.topk_groups == int(g["v3.topk_groups"])
        assert c.route_scale == float(g["v3.route_scale"]) and c.score == g["v3.score"]
    assert configs.V3_DECODE_FP8.weight == g["v3.weight"]
    c = configs.V2_BF16
    assert (c.dim, c.n_routed, c.top_k, c.n_shared) == (
        int(g["v2.dim"]), int(g["v2.n_routed"]), int(g["v2.top_k"]), int(g["v2.n_shared"]))


# ---------------------------------------------------------------- FFN closed forms
def test_swiglu_closed_form_permutations():
    """W1 = a*Id, W3 = b*P, W2 = Q (P, Q permutations, dim = I):
    FFN(u)_Q(i) = silu(a u_i) * b u_P(i), elementwise with math.exp."""
    n = 6
    P = np.eye(n)[[2, 0, 1, 5, 3, 4]]
    Q = np.eye(n)[[1, 3, 5, 0, 2, 4]]
    a, b = 1.5, -0.75
    w13 = np.vstack([a * np.eye(n), b * P])
    u = np.array([[0.3, -1.2, 2.0, 0.0, -0.4, 1.1]])
    got = oracle.swiglu_ffn(u, w13, Q)[0]
    h = np.array([(a * u[0, i]) / (1.0 + math.exp(-a * u[0, i])) * b * (P @ u[0])[i] for i in range(n)])
    want = Q @ h
    assert np.allclose(got, want, rtol=0, atol=1e-15)


def test_swiglu_preacts_unit_inputs_pick_columns():
    """u = e_j gives a = column j of W1 and c = column j of W3 (W13 = [W1; W3], rows
    first the gate half); a sum of two unit inputs gives the sum of the columns."""
    rng = np.random.default_rng(11)
    D, I = 7, 4
    w13 = rng.normal(size=(2 * I, D))
    for j in range(D):
        a, c = oracle.swiglu_preacts(np.eye(D)[j:j + 1], w13)
        assert np.array_equal(a[0], w13[:I, j]) and np.array_equal(c[0], w13[I:, j])
    a, c = oracle.swiglu_preacts((np.eye(D)[1] + np.eye(D)[5])[None], w13)
    assert np.allclose(a[0], w13[:I, 1] + w13[:I, 5], rtol=0, atol=1e-15)
    assert np.allclose(c[0], w13[I:, 1] + w13[I:, 5], rtol=0, atol=1e-15)


def test_swiglu_brute_force_loops():
    rng = np.random.default_rng(4)
    D, I = 5, 3
    u = rng.normal(size=(2, D))
    w13, w2 = rng.normal(size=(2 * I, D)), rng.normal(size=(D, I))
    got = oracle.swiglu_ffn(u, w13, w2)
    for t in range(2):
        h = []
        for i in range(I):
            a = math.fsum(w13[i, j] * u[t, j] for j in range(D))
            c = math.fsum(w13[I + i, j] * u[t, j] for j in range(D))
            h.append(a / (1.0 + math.exp(-a)) * c)
        for d in range(D):
            assert abs(got[t, d] - math.fsum(w2[d, i] * h[i] for i in range(I))) < 1e-13


def test_shared_split_identity():
    """S shared experts of hidden I = one SwiGLU of hidden S*I over stacked units."""
    rng = np.random.default_rng(6)
    D, I = 9, 4
    u = rng.normal(size=(5, D))
    parts = [(rng.normal(size=(2 * I, D)), rng.normal(size=(D, I))) for _ in range(2)]
    w13 = np.vstack([parts[0][0][:I], parts[1][0][:I], parts[0][0][I:], parts[1][0][I:]])
    w2 = np.hstack([parts[0][1], parts[1][1]])
    fused = oracle.swiglu_ffn(u, w13, w2)
    split = sum(oracle.swiglu_ffn(u, a, b) for a, b in parts)
    assert np.allclose(fused, split, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- layer invariants
def _random_layer(rng, T=48, D=24, E=16, I=8, S=1, G=4, TG=2, K=4, score="sigmoid", bias=True,
                  rs=2.5, norm=-1):
    spec = Spec(n_routed=E, n_groups=G, topk_groups=TG, top_k=K, score=score, route_scale=rs,
                norm_topk=norm)
    x = rng.normal(size=(T, D))
    wg = rng.normal(size=(E, D)) / math.sqrt(D)
    b = rng.uniform(-0.1, 0.1, size=E) if bias else None
    experts = [(rng.normal(size=(2 * I, D)) / math.sqrt(D), rng.normal(size=(D, I)) / math.sqrt(I))
               for _ in range(E)]
    shared = (rng.normal(size=(2 * S * I, D)) / math.sqrt(D),
              rng.normal(size=(D, S * I)) / math.sqrt(S * I)) if S else None
    return spec, x, wg, b, experts, shared


def test_groups_invariant_v3_constants():
    """Chosen experts lie in at most topk_groups groups, and those are top-scoring groups."""
    rng = np.random.default_rng(11)
    spec = Spec(n_routed=256, n_groups=8, topk_groups=4, top_k=8, score="sigmoid", route_scale=2.5)
    key = oracle.sigmoid(rng.normal(size=(500, 256))) + rng.uniform(-0.05, 0.05, size=256)
    idx = oracle.select_experts(key, spec, has_bias=True)
    gs = oracle.group_scores(key, 8, top2=True)
    for t in range(500):
        groups = set((idx[t] // 32).tolist())
        assert len(groups) <= 4
        fourth = np.sort(gs[t])[::-1][3]
        assert all(gs[t, j] >= fourth for j in groups)


def test_sigmoid_weights_sum_to_route_scale():
    rng = np.random.default_rng(12)
    spec, x, wg, b, _, _ = _random_layer(rng, T=300)
    res = oracle.gate(x, wg, b, spec)
    assert np.allclose(res.w.sum(axis=1), 2.5, rtol=1e-12, atol=0)
    assert (np.diff(res.idx, axis=1) > 0).all()          # ascending, distinct


def test_bias_steers_selection_but_not_weights():
    rng = np.random.default_rng(13)
    spec, x, wg, b, _, _ = _random_layer(rng, T=64, G=1, TG=1)
    b = np.zeros(16)
    b[5] = 10.0            # expert 5 always wins the ranking
    res = oracle.gate(x, wg, b, spec)
    assert (res.idx == 5).any(axis=1).all()
    s = oracle.sigmoid(oracle.gate_logits(x, wg))
    chosen = np.take_along_axis(s, res.idx, axis=1)
    assert np.allclose(res.w, 2.5 * chosen / chosen.sum(axis=1, keepdims=True), rtol=1e-14)


def test_identical_experts_closed_form():
    """All routed experts equal -> out = u + z + (sum of weights) FFN_0(u) = u + z + rs FFN_0(u)."""
    rng = np.random.default_rng(14)
    spec, x, wg, b, experts, shared = _random_layer(rng, T=40)
    same = experts[0]
    out, res = oracle.moe_layer(x, wg, b, lambda e: same, shared, spec)
    ffn0 = oracle.swiglu_ffn(x, *same)
    z = oracle.swiglu_ffn(x, *shared)
    assert np.allclose(out, x + z + 2.5 * ffn0, rtol=0, atol=1e-12)


def test_layer_terms_and_reductions():
    rng = np.random.default_rng(15)
    spec, x, wg, b, experts, shared = _random_layer(rng, T=32)
    full, res = oracle.moe_layer(x, wg, b, experts.__getitem__, shared, spec)
    # zero routed down-projections -> out = u + z
    zero_r = [(w13, np.zeros_like(w2)) for w13, w2 in experts]
    out, _ = oracle.moe_layer(x, wg, b, zero_r.__getitem__, shared, spec)
    assert np.allclose(out, x + oracle.swiglu_ffn(x, *shared), rtol=0, atol=1e-13)
    # no shared expert -> out = u + routed
    out_ns, _ = oracle.moe_layer(x, wg, b, experts.__getitem__, None, spec)
    assert np.allclose(full - out_ns, oracle.swiglu_ffn(x, *shared), rtol=0, atol=1e-12)
    # residual off -> out loses exactly u
    spec_nr = Spec(**{**spec.__dict__, "add_residual": 0})
    out_nr, _ = oracle.moe_layer(x, wg, b, experts.__getitem__, shared, spec_nr)
    assert np.allclose(full - out_nr, x, rtol=0, atol=1e-12)
    # routed term per token = explicit sum over its chosen experts
    for t in (0, 7, 31):
        r = sum(res.w[t, k] * oracle.swiglu_ffn(x[t:t + 1], *experts[res.idx[t, k]])[0] for k in range(4))
        assert np.allclose(out_ns[t] - x[t], r, rtol=0, atol=1e-12)
    # token subset gives the same rows
    sub, _ = oracle.moe_layer(x, wg, b, experts.__getitem__, shared, spec, tokens=[3, 17, 9])
    assert np.allclose(sub, full[[3, 17, 9]], rtol=0, atol=1e-13)


def test_group_reductions():
    rng = np.random.default_rng(16)
    key = rng.normal(size=(200, 16))
    plain = Spec(n_routed=16, n_groups=1, topk_groups=1, top_k=4, score="sigmoid", route_scale=1.0)
    all_groups = Spec(n_routed=16, n_groups=4, topk_groups=4, top_k=4, score="sigmoid", route_scale=1.0)
    for top2 in (False, True):
        assert np.array_equal(oracle.select_experts(key, plain, top2),
                              oracle.select_experts(key, all_groups, top2))


def test_dense_mixture_reductions():
    rng = np.random.default_rng(17)
    # sigmoid, top_k = E, renormalised: w = rs * s / sum(s)
    spec, x, wg, b, _, _ = _random_layer(rng, T=20, E=8, G=1, TG=1, K=8)
    res = oracle.gate(x, wg, b, spec)
    s = oracle.sigmoid(oracle.gate_logits(x, wg))
    assert np.allclose(res.w, 2.5 * s / s.sum(axis=1, keepdims=True), rtol=1e-14)
    # softmax, top_k = E, no renormalisation: weights are the probabilities (sum 1)
    spec = Spec(n_routed=8, n_groups=1, topk_groups=1, top_k=8, score="softmax", route_scale=1.0)
    res = oracle.gate(x, wg, None, spec)
    assert np.allclose(res.w.sum(axis=1), 1.0, rtol=1e-14)
    # softmax top-k weights are the full-softmax probabilities of the chosen experts
    spec = Spec(n_routed=8, n_groups=1, topk_groups=1, top_k=3, score="softmax", route_scale=1.0)
    res = oracle.gate(x, wg, None, spec)
    l = oracle.gate_logits(x, wg)
    for t in range(20):
        den = math.fsum(math.exp(v) for v in l[t])
        for k in range(3):
            assert abs(res.w[t, k] - math.exp(l[t, res.idx[t, k]]) / den) < 1e-14
        assert set(res.idx[t].tolist()) == set(np.argsort(-l[t], kind="stable")[:3].tolist())


def test_force_idx_keeps_step5_weights():
    rng = np.random.default_rng(18)
    spec, x, wg, b, experts, shared = _random_layer(rng, T=8)
    forced = np.array([[0, 1, 2, 3]] * 8)
    res = oracle.gate(x, wg, b, spec, force_idx=forced)
    s = oracle.sigmoid(oracle.gate_logits(x, wg))[:, :4]
    assert np.allclose(res.w, 2.5 * s / s.sum(axis=1, keepdims=True), rtol=1e-14)
