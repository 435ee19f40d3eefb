"""Pins for the bias-update oracle (auxiliary-loss-free balancing).

Against: a hand-worked example (tests/golden), the behaviour the pages state
(overloaded experts lose bias, underloaded ones gain it, and repeating the step
balances the experts' loads), exact handling of a fractional mean, and a
counting definition of the loads.  A flipped sign, a wrong mean (T instead of
T*K, or E instead of T*K/E) or an update applied to balanced experts fails one
of them.
"""
import os

import numpy as np

import oracle
from oracle import balance
from oracle import Spec

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _fixture(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = (s.strip() for s in line.split("=", 1))
                vals[k] = v
    return vals


def test_golden_bias_update():
    g = _fixture("bias_update_worked_example.txt")
    loads = np.array([int(v) for v in g["loads"].split()])
    bias = np.array([float(v) for v in g["bias"].split()], dtype=np.float32)
    want = np.array([float(v) for v in g["expect"].split()], dtype=np.float32)
    got = balance.bias_update(bias, loads, int(g["T"]), int(g["top_k"]), float(g["gamma"]))
    assert got.dtype == np.float32
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_loads_count_pairs():
    rng = np.random.default_rng(5)
    for _ in range(50):
        E, T, K = int(rng.integers(2, 20)), int(rng.integers(1, 30)), int(rng.integers(1, 4))
        idx = rng.integers(0, E, size=(T, K))
        loads = balance.expert_loads(idx, E)
        for e in range(E):   # counting definition, one pair at a time
            assert loads[e] == sum(1 for t in range(T) for k in range(K) if idx[t, k] == e)
        assert loads.sum() == T * K


def test_direction_and_balanced_experts():
    rng = np.random.default_rng(6)
    for _ in range(200):
        E, T, K = int(rng.integers(2, 40)), int(rng.integers(1, 200)), int(rng.integers(1, 9))
        loads = rng.multinomial(T * K, np.ones(E) / E)
        bias = rng.uniform(-0.1, 0.1, E).astype(np.float32)
        gamma = float(rng.choice([2.0 ** -10, 1e-3, 0.0]))
        new = balance.bias_update(bias, loads, T, K, gamma)
        mean = T * K / E
        for e in range(E):
            if loads[e] == mean:
                assert new[e].view(np.uint32) == bias[e].view(np.uint32)
            elif gamma == 0.0:
                assert new[e] == bias[e]
            elif loads[e] > mean:
                assert new[e] < bias[e] and abs(float(new[e]) - (float(bias[e]) - gamma)) <= 1e-7
            else:
                assert new[e] > bias[e] and abs(float(new[e]) - (float(bias[e]) + gamma)) <= 1e-7


def test_fractional_mean_is_exact():
    # T*K = 4 pairs over E = 3 experts: mean 4/3, so load 1 is under and load 2 is over
    new = balance.bias_update(np.zeros(3, np.float32), np.array([2, 1, 1]), 2, 2, 0.5)
    assert list(new) == [-0.5, 0.5, 0.5]
    # a mean that is an integer only after the product T*K: 3 tokens x 4 slots over 6 experts
    new = balance.bias_update(np.zeros(6, np.float32), np.array([2, 2, 2, 3, 1, 2]), 3, 4, 1.0)
    assert list(new) == [0.0, 0.0, 0.0, -1.0, 1.0, 0.0]


def test_repeated_updates_balance_the_experts():
    """The pages' purpose: with the bias steering selection, repeating the update
    evens out the experts' loads on a router that prefers a few experts."""
    rng = np.random.default_rng(7)
    E, T, K, D = 16, 256, 2, 32
    spec = Spec(n_routed=E, n_groups=1, topk_groups=1, top_k=K, score="sigmoid", route_scale=1.0)
    x = rng.standard_normal((T, D))
    w = rng.standard_normal((E, D)) * 0.05
    w[:3] += 0.2 * x.mean(axis=0) / np.linalg.norm(x.mean(axis=0))   # experts 0-2 favoured
    x = x + 3.0 * x.mean(axis=0)
    bias = np.zeros(E, np.float32)

    def imbalance(b):
        res = oracle.gate(x, w, b.astype(np.float64), spec)
        loads = balance.expert_loads(res.idx, E)
        return loads, loads.max() / (T * K / E)

    loads, start = imbalance(bias)
    assert start > 2.0
    for _ in range(300):
        bias = balance.bias_update(bias, loads, T, K, 2e-3)
        loads, _ = imbalance(bias)
    _, end = imbalance(bias)
    assert end < 0.5 * start and end < 1.6


def test_golden_sequence_balance_loss():
    g = _fixture("balance_loss_worked_example.txt")
    logits = np.array([[float(v) for v in g["logit0"].split()], [float(v) for v in g["logit1"].split()]])
    a = float(g["alpha"])
    split = balance.sequence_balance_loss(logits, np.array([[0], [1]]), "softmax", a, 2)
    same = balance.sequence_balance_loss(logits, np.array([[0], [0]]), "softmax", a, 2)
    assert np.isclose(split[0], float(g["expect_split"]), rtol=1e-12)
    assert np.isclose(same[0], float(g["expect_same"]), rtol=1e-12)


def test_balance_loss_closed_forms():
    # equal scores and perfectly balanced routing: f_i = 1, P_i = 1/E -> L = alpha
    E, K, T = 16, 4, 64
    idx = (np.arange(T * K) % E).reshape(T, K)
    for score in ("sigmoid", "softmax"):
        loss = balance.sequence_balance_loss(np.zeros((T, E)), idx, score, 0.01, T)
        assert np.isclose(loss[0], 0.01, rtol=1e-12)
    # every token on the same K experts with equal scores: f = E/K on those, L = alpha * E/K * K/E... = alpha
    # (sum of P over the chosen experts is K/E); a skewed score profile matched to the routing costs more
    idx1 = np.tile(np.arange(K), (T, 1))
    assert np.isclose(balance.sequence_balance_loss(np.zeros((T, E)), idx1, "softmax", 1.0, T)[0], 1.0)
    skew = np.zeros((T, E))
    skew[:, :K] = 2.0
    assert balance.sequence_balance_loss(skew, idx1, "softmax", 1.0, T)[0] > 1.5


def test_balance_loss_sequences_are_independent_and_relabeling_invariant():
    rng = np.random.default_rng(8)
    E, K, S = 12, 3, 40
    l = rng.standard_normal((2 * S, E))
    idx = np.stack([rng.choice(E, K, replace=False) for _ in range(2 * S)])
    both = balance.sequence_balance_loss(l, idx, "sigmoid", 0.1, S)
    first = balance.sequence_balance_loss(l[:S], idx[:S], "sigmoid", 0.1, S)
    second = balance.sequence_balance_loss(l[S:], idx[S:], "sigmoid", 0.1, S)
    assert np.allclose(both, [first[0], second[0]], rtol=1e-13)
    perm = rng.permutation(E)
    inv = np.argsort(perm)
    relabel = balance.sequence_balance_loss(l[:, perm], inv[idx], "sigmoid", 0.1, 2 * S)
    assert np.isclose(relabel[0], balance.sequence_balance_loss(l, idx, "sigmoid", 0.1, 2 * S)[0],
                      rtol=1e-12)
    # the score is normalised per token: adding a constant to a token's softmax logits changes nothing
    l2 = l + rng.standard_normal((2 * S, 1))
    assert np.allclose(balance.sequence_balance_loss(l2, idx, "softmax", 0.1, S),
                       balance.sequence_balance_loss(l, idx, "softmax", 0.1, S), rtol=1e-12)
