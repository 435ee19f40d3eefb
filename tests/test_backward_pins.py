"""Pins of the backward oracle (oracle/backward.py), independent of its code.

Every gradient is checked against central finite differences of the forward
oracle (itself pinned by test_oracle_pins.py): for L = sum <dout, out> and a
random direction v of one input, <dL/dtheta, v> must match
(L(theta + eps v) - L(theta - eps v)) / (2 eps).  The selection is held at the
unperturbed one (force_idx), as the gradient is defined almost everywhere and
the top-k is piecewise constant; the inputs have clear selection margins, so
the held selection is also the one the perturbed forward would make.

Invariants that a wrong sign or a missing term breaks:
  * renormalised weights are invariant to scaling the chosen scores, so the
    score gradient is orthogonal to them: sum_k ds_{e_k} s_{e_k} = 0;
  * softmax is invariant to adding a constant to a token's logits, so the
    logit gradient sums to zero per token;
  * with plain (not renormalised) weights, ds at a chosen expert is route_scale
    times dL/dw.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from oracle import backward as bw


def _layer(seed, T=6, D=8, E=8, G=2, TG=1, K=2, I=4, S=1, score="sigmoid", norm=-1, bias=True,
           residual=1):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, D))
    wg = rng.standard_normal((E, D)) / np.sqrt(D)
    b = rng.uniform(-0.1, 0.1, E) if bias else None
    w13 = rng.standard_normal((E, 2 * I, D)) / np.sqrt(D)
    w2 = rng.standard_normal((E, D, I)) / np.sqrt(I)
    sh = (rng.standard_normal((2 * S * I, D)) / np.sqrt(D), rng.standard_normal((D, S * I)) / np.sqrt(S * I)) if S else None
    spec = oracle.Spec(n_routed=E, n_groups=G, topk_groups=TG, top_k=K, score=score, route_scale=2.5,
                       norm_topk=norm, add_residual=residual)
    dout = rng.standard_normal((T, D))
    return dict(x=x, wg=wg, b=b, w13=w13, w2=w2, sh=sh, spec=spec, dout=dout, rng=rng)


def _loss(L, force_idx, x=None, wg=None, w13=None, w2=None, sh=None):
    x = L["x"] if x is None else x
    wg = L["wg"] if wg is None else wg
    w13 = L["w13"] if w13 is None else w13
    w2 = L["w2"] if w2 is None else w2
    sh = L["sh"] if sh is None else sh
    out, _ = oracle.moe_layer(x, wg, L["b"], lambda e: (w13[e], w2[e]), sh, L["spec"], force_idx=force_idx)
    return float((L["dout"] * out).sum())


CASES = [
    dict(score="sigmoid"),                                  # V3: sigmoid, renormalised, bias, groups
    dict(score="sigmoid", norm=0, bias=False, G=1, TG=1),   # sigmoid without renormalisation
    dict(score="softmax", bias=False, G=1, TG=1),           # V2-Lite style: softmax, plain weights
    dict(score="softmax", norm=1, G=4, TG=2, K=3),          # softmax renormalised, with bias
    dict(score="sigmoid", S=0, residual=0),                 # no shared expert, no residual
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_gradients_match_finite_differences(case):
    L = _layer(100 + case, **CASES[case])
    g = bw.moe_layer_backward(L["x"], L["wg"], L["b"], lambda e: (L["w13"][e], L["w2"][e]), L["sh"],
                              L["spec"], L["dout"])
    idx = g.gate.idx
    eps = 1e-6
    rng = L["rng"]

    def check(name, grad, **kw):
        key, base = next(iter(kw.items()))
        v = rng.standard_normal(base.shape)
        fd = (_loss(L, idx, **{key: base + eps * v}) - _loss(L, idx, **{key: base - eps * v})) / (2 * eps)
        an = float((grad * v).sum())
        assert abs(an - fd) <= 1e-6 * max(1.0, abs(fd)), (name, an, fd)

    check("dx", g.dx, x=L["x"])
    check("dw_gate", g.dw_gate, wg=L["wg"])
    full13 = np.zeros_like(L["w13"])
    full2 = np.zeros_like(L["w2"])
    for e, v in g.dw13.items():
        full13[e] = v
    for e, v in g.dw2.items():
        full2[e] = v
    check("dw13", full13, w13=L["w13"])
    check("dw2", full2, w2=L["w2"])
    if L["sh"] is not None:
        s13, s2 = L["sh"]
        v13 = rng.standard_normal(s13.shape)
        for name, grad, pert in (("dsw13", g.dsw13, lambda t: (s13 + t * v13, s2)),):
            fd = (_loss(L, idx, sh=pert(eps)) - _loss(L, idx, sh=pert(-eps))) / (2 * eps)
            assert abs(float((grad * v13).sum()) - fd) <= 1e-6 * max(1.0, abs(fd)), name
        v2 = rng.standard_normal(s2.shape)
        fd = (_loss(L, idx, sh=(s13, s2 + eps * v2)) - _loss(L, idx, sh=(s13, s2 - eps * v2))) / (2 * eps)
        assert abs(float((g.dsw2 * v2).sum()) - fd) <= 1e-6 * max(1.0, abs(fd))


def test_selection_held_matches_free_selection():
    """With these margins the perturbed forward picks the same experts, so holding
    the selection in the finite differences does not change the function."""
    L = _layer(7)
    g = oracle.gate(L["x"], L["wg"], L["b"], L["spec"])
    assert g.expert_gap.min() > 1e-4 and g.group_gap.min() > 1e-4
    v = L["rng"].standard_normal(L["x"].shape)
    for t in (1e-6, -1e-6):
        g2 = oracle.gate(L["x"] + t * v, L["wg"], L["b"], L["spec"])
        assert np.array_equal(g2.idx, g.idx)


def test_renormalised_score_gradient_is_orthogonal_to_the_scores():
    rng = np.random.default_rng(3)
    spec = oracle.Spec(n_routed=16, n_groups=1, topk_groups=1, top_k=4, score="sigmoid", route_scale=2.5)
    s = rng.uniform(0.05, 0.95, (5, 16))
    idx = np.sort(np.stack([rng.permutation(16)[:4] for _ in range(5)]), axis=-1)
    dw = rng.standard_normal((5, 4))
    ds = bw.route_weights_backward(s, idx, dw, spec)
    sel = np.take_along_axis(s, idx, -1)
    assert np.allclose((np.take_along_axis(ds, idx, -1) * sel).sum(-1), 0.0, atol=1e-12)
    mask = np.ones_like(s, dtype=bool)
    np.put_along_axis(mask, idx, False, axis=-1)
    assert np.all(ds[mask] == 0.0)


def test_plain_weights_gradient_is_route_scale_times_dw():
    rng = np.random.default_rng(4)
    spec = oracle.Spec(n_routed=8, n_groups=1, topk_groups=1, top_k=2, score="softmax", route_scale=1.5)
    s = rng.uniform(0.0, 0.3, (3, 8))
    idx = np.array([[0, 5], [2, 3], [1, 7]])
    dw = rng.standard_normal((3, 2))
    ds = bw.route_weights_backward(s, idx, dw, spec)
    assert np.allclose(np.take_along_axis(ds, idx, -1), 1.5 * dw, rtol=0, atol=1e-15)


def test_softmax_logit_gradient_sums_to_zero():
    rng = np.random.default_rng(5)
    l = rng.standard_normal((4, 10))
    s, _ = oracle.gate_scores(l, "softmax", None)
    dl = bw.gate_scores_backward(s, rng.standard_normal((4, 10)), "softmax")
    assert np.allclose(dl.sum(-1), 0.0, atol=1e-14)


def test_swiglu_backward_scalar_closed_form():
    """One unit, one input: y = w2 * silu(w1 u) * (w3 u); compare every partial
    derivative with its hand-derived closed form at a point."""
    u, w1, w3, w2 = 0.7, -1.3, 0.4, 2.0
    a, c = w1 * u, w3 * u
    sg = 1.0 / (1.0 + np.exp(-a))
    dsilu = sg * (1.0 + a * (1.0 - sg))
    du, dw13, dw2 = bw.swiglu_ffn_backward(np.array([[u]]), np.array([[w1], [w3]]), np.array([[w2]]),
                                           np.array([[1.0]]))
    assert np.isclose(dw2[0, 0], a * sg * c)
    assert np.isclose(dw13[0, 0], w2 * c * dsilu * u)
    assert np.isclose(dw13[1, 0], w2 * a * sg * u)
    assert np.isclose(du[0, 0], w2 * (c * dsilu * w1 + a * sg * w3))
