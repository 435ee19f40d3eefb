"""Pins for the fp8 W8A8 oracle: the e4m3 encoder, the 1x128 activation
quantiser and the layer with both expert GEMMs in fp8.

Against: the format's decoder on every code, rounding ties and saturation by
hand, torch's e4m3 cast, a hand-worked quantisation and a hand-worked W8A8
SwiGLU FFN (tests/golden), the quantiser's error bound, the per-token
independence of 1x128 blocks, and the identical-experts closed form of the
layer.  Planted slips in the FFN (x or h left unquantised, a and c quantised
in place of h, blocks taken along tokens instead of along a row) each fail at
least one of these pins.
"""
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import Spec
from oracle import w8a8

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


def test_encode_roundtrips_every_code():
    c = np.arange(256, dtype=np.uint8)
    v = oracle.decode_e4m3(c)
    ok = ~np.isnan(v)
    assert np.array_equal(w8a8.encode_e4m3(v[ok]), c[ok])
    assert w8a8.encode_e4m3(np.array([np.nan]))[0] & 0x7F == 0x7F


def test_encode_ties_to_even_and_saturates():
    # 1.0625 lies halfway between 1.0 (m=0) and 1.125 (m=1): even mantissa 0 wins
    assert w8a8.encode_e4m3(np.array([1.0625]))[0] == 0x38
    # 1.1875 halfway between 1.125 (m=1) and 1.25 (m=2): m=2
    assert w8a8.encode_e4m3(np.array([1.1875]))[0] == 0x3A
    # 15.5 halfway between 15 (E=10, m=7) and 16 (E=11, m=0): carries into the exponent
    assert w8a8.encode_e4m3(np.array([15.5]))[0] == 0x58
    # subnormals are multiples of 2^-9: half of 2^-9 rounds to 0, 1.5 units to 2
    assert w8a8.encode_e4m3(np.array([2.0 ** -10]))[0] == 0x00
    assert w8a8.encode_e4m3(np.array([1.5 * 2.0 ** -9]))[0] == 0x02
    # saturation at +-448
    assert list(w8a8.encode_e4m3(np.array([448.0, 460.0, 1e9, -1e9]))) == [0x7E, 0x7E, 0x7E, 0xFE]


def test_encode_matches_torch_cast_in_range():
    r = np.random.default_rng(3).standard_normal(200_000).astype(np.float32)
    r = np.concatenate([r * 100, r * 1e-3, r * 1e-2])
    t = torch.from_numpy(r).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(w8a8.encode_e4m3(r), t)


def test_golden_activation_quant():
    g = _fixture("fp8_act_quant_worked_example.txt")
    a = np.zeros((1, 128), np.float32)
    a[0, :3] = [3.5, -1.75, 0.3]
    codes, s = w8a8.quant_1x128(a)
    assert s.dtype == np.float32 and s[0, 0] == float(g["scale"])
    assert [int(c) for c in codes[0, :3]] == [int(v, 16) for v in g["codes"].split()]
    assert not codes[0, 3:].any()
    deq = w8a8.dequant_1x128(codes, s)
    assert list(deq[0, :3]) == [float(v) for v in g["dequant"].split()]


def test_quant_block_properties():
    rng = np.random.default_rng(4)
    a = (rng.standard_normal((64, 512)) * np.exp(rng.uniform(-8, 8, (64, 1)))).astype(np.float32)
    a[3, 128:256] = 0.0                                  # an all-zero block
    codes, s = w8a8.quant_1x128(a)
    assert s.shape == (64, 4) and s[3, 1] == 1.0 and not codes[3, 128:256].any()
    blk = np.abs(a).reshape(64, 4, 128)
    arg = blk.argmax(axis=2)
    for r in range(64):
        for b in range(4):
            if s[r, b] != 1.0 or blk[r, b].max() > 0:
                assert codes[r, b * 128 + arg[r, b]] & 0x7F == 0x7E   # the block max maps to 448
    deq = w8a8.dequant_1x128(codes, s)
    # round to nearest with 3 mantissa bits: relative error <= 2^-4 for normal codes,
    # absolute <= 2^-10 * s below the normal range
    err = np.abs(deq - a.astype(np.float64))
    bound = np.maximum(np.abs(a) * 2.0 ** -4, np.repeat(s, 128, axis=1) * 2.0 ** -10) * (1 + 1e-6)
    assert (err <= bound).all()


def test_layer_identical_experts_closed_form():
    rng = np.random.default_rng(5)
    T, D, E, I, K = 6, 256, 8, 128, 2
    spec = Spec(n_routed=E, n_groups=1, topk_groups=1, top_k=K, score="sigmoid", route_scale=2.5)
    x = rng.standard_normal((T, D))
    wg = rng.standard_normal((E, D)) / 16
    w13 = rng.standard_normal((2 * I, D)) / 16
    w2 = rng.standard_normal((D, I)) / 11
    s13 = rng.standard_normal((2 * I, D)) / 16
    s2 = rng.standard_normal((D, I)) / 11
    out, g = w8a8.moe_layer_w8a8(x, wg, None, lambda e: (w13, w2), (s13, s2), spec)
    want = x + w8a8.swiglu_ffn_w8a8(x, s13, s2) + 2.5 * w8a8.swiglu_ffn_w8a8(x, w13, w2)
    assert np.allclose(out, want, rtol=1e-12, atol=1e-12)
    # and it stays within fp8 quantisation error of the unquantised layer, but not equal to it
    ref, _ = oracle.moe_layer(x, wg, None, lambda e: (w13, w2), (s13, s2), spec)
    rel = np.abs(out - ref).max() / np.abs(ref).max()
    assert 1e-4 < rel < 5e-2


def test_h_is_quantised_before_the_down_projection():
    """A planted omission (down projection fed the unquantised h) must be visible."""
    rng = np.random.default_rng(6)
    x = rng.standard_normal((4, 256))
    w13 = rng.standard_normal((256, 256)) / 16
    w2 = rng.standard_normal((256, 128)) / 11
    got = w8a8.swiglu_ffn_w8a8(x, w13, w2)
    xa = w8a8.dequant_1x128(*w8a8.quant_1x128(x))
    h = oracle.silu(xa @ w13[:128].T) * (xa @ w13[128:].T)
    no_hq = h @ w2.T
    with_hq = w8a8.dequant_1x128(*w8a8.quant_1x128(h)) @ w2.T
    assert np.allclose(got, with_hq, rtol=1e-12, atol=1e-12)
    assert not np.allclose(got, no_hq, rtol=1e-6, atol=1e-9)


# ---------------------------------------------------------------------------
# The W8A8 SwiGLU FFN, pinned by a hand-worked example and by row independence
# ---------------------------------------------------------------------------
def _golden_ffn_inputs():
    """x [1, 128], W13 [256, 128], W2 [128, 128] as the worked example states them."""
    D = I = 128
    x = np.zeros((1, D))
    x[0, :2] = [3.5, 0.3]
    w13 = np.zeros((2 * I, D))
    w13[0, 0] = 1.0                       # W1[0] = e0
    w13[1, 1] = 1.0                       # W1[1] = e1
    w13[2, 0], w13[2, 1] = 0.5, 1.0       # W1[2] = 0.5 e0 + e1
    w13[I + 0, 1] = 1.0                   # W3[0] = e1
    w13[I + 1, 0] = 1.0                   # W3[1] = e0
    w13[I + 2, 0], w13[I + 2, 1] = 1.0, -2.0   # W3[2] = e0 - 2 e1
    w2 = np.zeros((D, I))
    w2[0, 0] = w2[1, 1] = w2[2, 2] = 1.0
    w2[3, :3] = [0.5, -1.0, 0.25]
    return x, w13, w2


def pin_golden_ffn(ffn) -> bool:
    g = _fixture("w8a8_ffn_worked_example.txt")
    x, w13, w2 = _golden_ffn_inputs()
    out = ffn(x, w13, w2)
    s_h = float(g["h_scale"])
    want = np.zeros(128)
    want[:4] = [float(v) * s_h for v in g["out_over_h_scale"].split()]
    return bool(np.allclose(out[0], want, rtol=1e-12, atol=1e-15))


def pin_rows_independent(ffn) -> bool:
    """1x128 blocks lie inside one token's row: a token's output cannot depend on the others."""
    rng = np.random.default_rng(8)
    T, D, I = 130, 256, 128
    x = rng.standard_normal((T, D)) * np.exp2(rng.integers(-8, 5, (T, 1)))
    w13 = rng.standard_normal((2 * I, D)) / 16
    w2 = rng.standard_normal((D, I)) / 11
    batch = ffn(x, w13, w2)
    alone = np.concatenate([ffn(x[t:t + 1], w13, w2) for t in (0, 1, 77, T - 1)])
    return bool(np.allclose(batch[[0, 1, 77, T - 1]], alone, rtol=1e-12, atol=0))


PINS = [pin_golden_ffn, pin_rows_independent]


def test_golden_w8a8_ffn_codes():
    """The quantiser's decisions of the worked example: x and h codes and scales."""
    g = _fixture("w8a8_ffn_worked_example.txt")
    x, w13, w2 = _golden_ffn_inputs()
    xc, xs = w8a8.quant_1x128(x)
    assert xs[0, 0] == float(g["x_scale"])
    assert [int(c) for c in xc[0, :2]] == [int(v, 16) for v in g["x_codes"].split()]
    xq = w8a8.dequant_1x128(xc, xs)
    h = oracle.silu(xq @ w13[:128].T) * (xq @ w13[128:].T)
    hc, hs = w8a8.quant_1x128(h)
    assert hs[0, 0] == np.float32(float(g["h_scale"]))
    assert [int(c) for c in hc[0, :3]] == [int(v, 16) for v in g["h_codes"].split()]
    assert not hc[0, 3:].any()


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_w8a8_ffn_meets_pin(pin):
    assert pin(w8a8.swiglu_ffn_w8a8)


def _quant_cols(a):
    """Blocks of 128 consecutive TOKENS of one column (a planted slip), zero-padded."""
    a = np.asarray(a, np.float64)
    T = a.shape[0]
    pad = (-T) % 128
    at = np.concatenate([a, np.zeros((pad, a.shape[1]))]).T
    return w8a8.dequant_1x128(*w8a8.quant_1x128(at)).T[:T]


def _q(a):
    return w8a8.dequant_1x128(*w8a8.quant_1x128(a))


def _slip_skip_x(x, w13, w2):
    H = w2.shape[1]
    return _q(oracle.silu(x @ w13[:H].T) * (x @ w13[H:].T)) @ w2.T


def _slip_skip_h(x, w13, w2):
    H = w2.shape[1]
    xa = _q(x)
    return (oracle.silu(xa @ w13[:H].T) * (xa @ w13[H:].T)) @ w2.T


def _slip_quant_a_c(x, w13, w2):
    H = w2.shape[1]
    xa = _q(x)
    return (oracle.silu(_q(xa @ w13[:H].T)) * _q(xa @ w13[H:].T)) @ w2.T


def _slip_h_transposed(x, w13, w2):
    H = w2.shape[1]
    xa = _q(x)
    return _quant_cols(oracle.silu(xa @ w13[:H].T) * (xa @ w13[H:].T)) @ w2.T


def _slip_x_transposed(x, w13, w2):
    H = w2.shape[1]
    xa = _quant_cols(x)
    return _q(oracle.silu(xa @ w13[:H].T) * (xa @ w13[H:].T)) @ w2.T


@pytest.mark.parametrize("slip", [_slip_skip_x, _slip_skip_h, _slip_quant_a_c, _slip_h_transposed,
                                  _slip_x_transposed], ids=lambda f: f.__name__)
def test_planted_slip_fails_a_pin(slip):
    failed = [p.__name__ for p in PINS if not p(slip)]
    assert failed, f"{slip.__name__} passes every pin"
