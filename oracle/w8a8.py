"""Oracle: the DeepSeekMoE layer with fp8 (e4m3) weights AND fp8 activations.

TEST INFRASTRUCTURE.  Only the tests, the smoke check of the package entry file
and the CPU-baseline leg of the benchmark may import this module.  The library
never imports it and shares no code with it.

What is computed, and where the pages state it
----------------------------------------------
  * DeepSeek-V3 notes page (73biji.xyz/llm_pp_dsv3), "DeepSeek-V3 (model.py
    config)" table: the released layer runs its experts in fp8.
  * DeepSeek-R1 analysis page (deepseek.csdn.net), training-process
    hyper-parameters paragraph: training uses FP8 mixed precision (W8A8), i.e.
    both the weights and the activations entering the matrix products are
    8-bit floats.
  * Everything else (gate, SwiGLU experts, shared expert, combine) is the layer
    of moe_oracle.py, unchanged.

Readings where the pages are silent (also listed in the design notes):
  * format: OCP e4m3fn (max 448, S.1111.111 = NaN, no infinities); weights keep
    their 128 x 128 fp32 block scales; activations get one fp32 scale per row
    per 128 consecutive columns (1 x 128 blocks);
  * quantiser, in float32: s = max|a| / 448 over the block (1 for an all-zero
    block), code = round-to-nearest-even(a / s) in e4m3, saturating at 448;
  * activations are quantised right before each expert GEMM: x (exact in bf16)
    before gate/up, and the SwiGLU output h, rounded to float32, before down;
    the gate and the combine keep bf16/fp32 as in the bf16 layer;
  * products of codes and scales are exact in float64, so the oracle's only
    roundings are the quantisers' own decisions.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from .moe_oracle import (Spec, decode_e4m3, gate, silu)

E4M3_MAX = 448.0
BLOCK = 128


def encode_e4m3(v: np.ndarray) -> np.ndarray:
    """float values -> OCP e4m3fn codes, round to nearest (ties to even), saturating.

    Normal numbers are (1 + m/8) * 2^(E-7) for E in 1..15 (E = 15, m = 7 is
    NaN); subnormals m/8 * 2^-6.  Magnitudes at or beyond 448 map to 448.
    """
    a = np.asarray(v, dtype=np.float64)
    nan = np.isnan(a)
    sign = (np.signbit(a)).astype(np.uint8) << 7
    mag = np.where(nan, 0.0, np.abs(a))
    out = np.zeros(a.shape, dtype=np.uint8)
    # subnormal range: multiples of 2^-9 below 2^-6
    sub = mag < 2.0 ** -6
    m_sub = np.rint(mag[sub] / 2.0 ** -9)          # 0..8; 8 becomes the smallest normal
    out[sub] = np.where(m_sub >= 8, 1 << 3, m_sub).astype(np.uint8)
    nrm = ~sub
    mn = np.minimum(mag[nrm], E4M3_MAX)
    e = np.floor(np.log2(mn)).astype(np.int64)
    # log2 of an exact power of two is exact; guard the floor against rounding anyway
    e = np.where(np.exp2(e) > mn, e - 1, e)
    e = np.where(np.exp2(e + 1) <= mn, e + 1, e)
    m = np.rint((mn / np.exp2(e) - 1.0) * 8.0)     # exact scaling; rint ties to even
    carry = m >= 8
    e = np.where(carry, e + 1, e)
    m = np.where(carry, 0, m)
    E = e + 7                                         # mn <= 448 = 1.75 * 2^8 keeps E <= 15, m <= 6
    out[nrm] = ((E << 3) | m.astype(np.int64)).astype(np.uint8)
    out = out | sign
    out[nan] = 0x7F
    return out


def quant_1x128(a: np.ndarray):
    """[R, C] values -> (codes uint8 [R, C], scales float32 [R, C/128]), decisions in float32."""
    a32 = np.asarray(a, dtype=np.float32)
    R, C = a32.shape
    assert C % BLOCK == 0, C
    blk = a32.reshape(R, C // BLOCK, BLOCK)
    amax = np.abs(blk).max(axis=2)
    s = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    q = (blk / s[:, :, None]).astype(np.float32)      # one float32 division per element
    return encode_e4m3(q).reshape(R, C), s


def dequant_1x128(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    q = decode_e4m3(codes)
    return q * np.repeat(np.asarray(scales, np.float64), BLOCK, axis=1)


def swiglu_ffn_w8a8(x: np.ndarray, w13: np.ndarray, w2: np.ndarray) -> np.ndarray:
    """FFN(x) = W2 q(silu(W1 q(x)) * (W3 q(x))) with q() the 1x128 activation quantiser.

    w13 [2H, D] and w2 [D, H] are the dequantised (exact) fp8 weights."""
    H = w2.shape[1]
    xa = dequant_1x128(*quant_1x128(x))
    a = xa @ w13[:H].T
    c = xa @ w13[H:].T
    h = silu(a) * c
    ha = dequant_1x128(*quant_1x128(h))
    return ha @ w2.T


def moe_layer_w8a8(x: np.ndarray, w_gate: np.ndarray, bias: Optional[np.ndarray], expert_w,
                   shared, spec: Spec, tokens=None, force_idx=None):
    """The layer output with both expert GEMMs in fp8 x fp8 (see the module doc).

    Same structure and summation order as moe_oracle.moe_layer: expert_w(e) ->
    (w13_e [2I, D], w2_e [D, I]) dequantised float64; shared is (sw13, sw2) or
    None; x holds the exact bf16 values as float64.  The quantiser works per
    token row, so a token's result does not depend on the other tokens."""
    x = np.asarray(x, np.float64)
    g = gate(x, w_gate, bias, spec, force_idx=force_idx)
    toks = np.arange(x.shape[0]) if tokens is None else np.asarray(tokens, dtype=np.int64)
    u = x[toks]
    routed = np.zeros_like(u)
    idx, w = g.idx[toks], g.w[toks]
    for e in np.unique(idx):               # ascending expert index, as the sum is ordered
        rows, slot = np.nonzero(idx == e)
        w13, w2 = expert_w(int(e))
        routed[rows] += w[rows, slot][:, None] * swiglu_ffn_w8a8(u[rows], w13, w2)
    out = routed
    if shared is not None:
        out = swiglu_ffn_w8a8(u, shared[0], shared[1]) + out
    if spec.add_residual:
        out = u + out
    return out, g
