"""Oracle: the forward pass of one DeepSeekMoE layer, in plain float64 NumPy.

TEST INFRASTRUCTURE.  Only the tests, the smoke check of the package entry file
and the CPU-baseline leg of the benchmark may import this module.  The library
(routed_expert_moe_amd) never imports it and shares no code with it; the two
meet only through the tensors drawn by the seeded input generator.

What is computed, and where the pages state it
----------------------------------------------
Pages cited ("DSV3 notes" = the DeepSeek-V3 notes page, 73biji.xyz/llm_pp_dsv3):
  * DSV3 notes, "DeepSeekMoE" paragraph: the conventional MoE ranks
    g' = Softmax(W_g u_t) and keeps the TopK; DeepSeekMoE adds shared experts
    that every token passes through, fine-grained experts, and sigmoid scoring
    in place of softmax; the layer output is
        h'_t = u_t + FFN_share(u_t) + sum_r g_{r,t} FFN_r(u_t).
  * DSV3 notes, "V3 improvement 1" (auxiliary-loss-free balancing): the ranked
    quantity is s_{i,t} + b_i; the bias decides selection only.
  * DSV3 notes, gate flow (five steps): sigmoid scores (+bias); split into
    n_groups, a group scores its max (no bias) or the sum of its two largest
    biased scores (bias); keep topk_groups groups, the others become -inf;
    global TopK; gather the ORIGINAL scores at the chosen experts, normalise
    and multiply by route_scale.
  * DSV3 notes, MoE forward (four steps): loop over experts adding
    expert(x[idx]) * w into y for the tokens that chose it, then add the shared
    expert's output z.
  * DSV3 notes, "DeepSeek-V3 (model.py config)" table: route_scale 2.5,
    8 groups keep 4, sigmoid scoring, fp8 weights.

Readings where the pages are silent (each is also listed in the design notes):
  * expert FFN = SwiGLU: FFN(u) = W2 (silu(W1 u) * (W3 u)), silu(a) = a*sigmoid(a);
    W13 stacks W1 rows [0, I) over W3 rows [I, 2I);
  * n_shared = S shared experts act as ONE SwiGLU of hidden size S*I (the sum of
    S FFNs equals one FFN over the concatenated hidden units);
  * softmax scoring runs over all experts; with no bias the ranked key is the
    logit itself (same order as the softmax probability), with a bias it is p+b;
    weights are p at the chosen experts, renormalised only if asked;
  * sigmoid scoring renormalises the chosen weights (norm_topk default);
  * ties rank the lower expert index (and the lower group index) first;
  * chosen experts are reported in ascending expert index; the routed sum runs
    in that order;
  * masked groups get -inf (keys may be negative once a bias is added);
  * the group score is the top-2 sum whenever a bias is given, else the max;
  * fp8 weights are OCP e4m3fn codes (no infinities, 0x7F/0xFF = NaN) times one
    fp32 scale per 128x128 block; the decoded product is exact in float64.

Everything here is float64 except `select_experts`, which ranks in whatever
floating type its keys arrive in (so it can replay a selection on float32 keys
exactly).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Callable, Optional, Sequence

import numpy as np


# --------------------------------------------------------------------------
# storage decoding (exact)
# --------------------------------------------------------------------------
def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64: the bf16 value is the top half of an fp32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    """OCP e4m3fn codes (uint8) -> float64 by the format's definition.

    bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0 mantissa;
    exponent 0 encodes subnormals m/8 * 2^-6; S.1111.111 is NaN; no infinities.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = (m / 8.0) * 2.0 ** -6
    v = np.where(e == 0, sub, normal)
    v = np.where((e == 15) & (c & 0x7 == 7), np.nan, v)
    return sign * v


def dequant_e4m3_block128(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """[R, C] e4m3 codes with [R/128, C/128] fp32 scales -> float64 [R, C] = q * s."""
    q = decode_e4m3(codes)
    s = np.asarray(scales, dtype=np.float64)
    s_full = np.repeat(np.repeat(s, 128, axis=0), 128, axis=1)
    return q * s_full


# --------------------------------------------------------------------------
# the layer's hyper-parameters
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class Spec:
    n_routed: int
    n_groups: int
    topk_groups: int
    top_k: int
    score: str               # "sigmoid" | "softmax"
    route_scale: float
    norm_topk: int = -1      # -1: sigmoid normalises, softmax does not
    add_residual: int = 1

    @property
    def normalise(self) -> bool:
        if self.norm_topk >= 0:
            return bool(self.norm_topk)
        return self.score == "sigmoid"


# --------------------------------------------------------------------------
# gate
# --------------------------------------------------------------------------
def sigmoid(z: np.ndarray) -> np.ndarray:
    # for z < -709, exp(-z) overflows to inf and 1 / (1 + inf) = 0 is the correctly rounded value
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def gate_logits(x: np.ndarray, w_gate: np.ndarray) -> np.ndarray:
    """l = x W_g^T: one logit per (token, routed expert)."""
    return np.asarray(x, np.float64) @ np.asarray(w_gate, np.float64).T


def gate_scores(logits: np.ndarray, score: str, bias: Optional[np.ndarray]):
    """Return (s, key): s feeds the weights, key is what the TopK ranks."""
    if score == "sigmoid":
        s = sigmoid(logits)
        key = s + bias[None, :] if bias is not None else s.copy()
    elif score == "softmax":
        z = logits - logits.max(axis=-1, keepdims=True)
        ez = np.exp(z)
        s = ez / ez.sum(axis=-1, keepdims=True)
        key = s + bias[None, :] if bias is not None else logits.copy()
    else:
        raise ValueError(score)
    return s, key


def group_scores(key: np.ndarray, n_groups: int, top2: bool) -> np.ndarray:
    """Per-group score: sum of the two largest keys (top2) or the largest key."""
    T, E = key.shape
    g = key.reshape(T, n_groups, E // n_groups)
    if top2:
        srt = np.sort(g, axis=-1)
        return srt[..., -1] + srt[..., -2]
    return g.max(axis=-1)


def _rank_desc(v: np.ndarray) -> np.ndarray:
    """Indices ordering the last axis by value descending, equal values by index ascending."""
    return np.argsort(-v, axis=-1, kind="stable")


def select_experts(key: np.ndarray, spec: Spec, has_bias: bool) -> np.ndarray:
    """Group-limited TopK on `key` [T, E]; returns the chosen experts [T, K], ascending.

    Ranks in the dtype of `key` (float64 in the forward; float32 to replay a
    selection on a GPU's exported keys).
    """
    T, E = key.shape
    masked = key
    if spec.n_groups > 1:
        gs = group_scores(key, spec.n_groups, top2=has_bias)
        keep = _rank_desc(gs)[:, : spec.topk_groups]
        group_on = np.zeros((T, spec.n_groups), dtype=bool)
        np.put_along_axis(group_on, keep, True, axis=-1)
        expert_on = np.repeat(group_on, E // spec.n_groups, axis=1)
        masked = np.where(expert_on, key, np.array(-np.inf, dtype=key.dtype))
    chosen = _rank_desc(masked)[:, : spec.top_k]
    return np.sort(chosen, axis=-1)


def selection_margins(key: np.ndarray, spec: Spec, has_bias: bool):
    """Gaps that a perturbation of the keys must close to change the selection.

    Returns (expert_gap [T], group_gap [T]): the K-th minus the (K+1)-th surviving
    key, and the topk_groups-th minus the next group score (inf where no
    competitor exists).
    """
    T, E = key.shape
    group_gap = np.full(T, np.inf)
    masked = key
    if spec.n_groups > 1:
        gs = group_scores(key, spec.n_groups, top2=has_bias)
        srt = -np.sort(-gs, axis=-1)
        if spec.topk_groups < spec.n_groups:
            group_gap = srt[:, spec.topk_groups - 1] - srt[:, spec.topk_groups]
        keep = _rank_desc(gs)[:, : spec.topk_groups]
        group_on = np.zeros((T, spec.n_groups), dtype=bool)
        np.put_along_axis(group_on, keep, True, axis=-1)
        masked = np.where(np.repeat(group_on, E // spec.n_groups, axis=1), key, -np.inf)
    srt = -np.sort(-masked, axis=-1)
    expert_gap = np.full(T, np.inf)
    if spec.top_k < E:
        nxt = srt[:, spec.top_k]
        expert_gap = np.where(np.isfinite(nxt), srt[:, spec.top_k - 1] - nxt, np.inf)
    return expert_gap, group_gap


def route_weights(s: np.ndarray, idx: np.ndarray, spec: Spec) -> np.ndarray:
    """Gather the unbiased scores at the chosen experts, renormalise if asked, scale."""
    w = np.take_along_axis(s, idx, axis=-1)
    if spec.normalise:
        w = w / w.sum(axis=-1, keepdims=True)
    return w * spec.route_scale


# --------------------------------------------------------------------------
# experts
# --------------------------------------------------------------------------
def silu(a: np.ndarray) -> np.ndarray:
    return a * sigmoid(a)


def swiglu_preacts(xr: np.ndarray, w13: np.ndarray):
    """The SwiGLU's two inputs for each row of xr: a = W1 u and c = W3 u, W13 = [W1; W3]."""
    inter = w13.shape[0] // 2
    return xr @ w13[:inter].T, xr @ w13[inter:].T


def swiglu_ffn(xr: np.ndarray, w13: np.ndarray, w2: np.ndarray) -> np.ndarray:
    """FFN(u) = W2 (silu(W1 u) * (W3 u)) for each row of xr; W13 = [W1; W3]."""
    a, c = swiglu_preacts(xr, w13)
    return (silu(a) * c) @ w2.T


# --------------------------------------------------------------------------
# the layer
# --------------------------------------------------------------------------
@dataclass
class GateResult:
    logits: np.ndarray       # [T, E]
    s: np.ndarray            # [T, E] unbiased scores (sigmoid or softmax probabilities)
    key: np.ndarray          # [T, E] ranked quantity
    idx: np.ndarray          # [T, K] chosen experts, ascending
    w: np.ndarray            # [T, K] routing weights
    expert_gap: np.ndarray   # [T]
    group_gap: np.ndarray    # [T]


def gate(x: np.ndarray, w_gate: np.ndarray, bias: Optional[np.ndarray], spec: Spec,
         force_idx: Optional[np.ndarray] = None) -> GateResult:
    """Gate steps 1-5.  `force_idx` replaces the selection (weights still follow step 5)."""
    l = gate_logits(x, w_gate)
    b = None if bias is None else np.asarray(bias, np.float64)
    s, key = gate_scores(l, spec.score, b)
    idx = select_experts(key, spec, has_bias=b is not None)
    eg, gg = selection_margins(key, spec, has_bias=b is not None)
    if force_idx is not None:
        idx = np.sort(np.asarray(force_idx, dtype=np.int64), axis=-1)
    w = route_weights(s, idx, spec)
    return GateResult(l, s, key, idx, w, eg, gg)


ExpertFn = Callable[[int], "tuple[np.ndarray, np.ndarray]"]


def moe_layer(x: np.ndarray, w_gate: np.ndarray, bias: Optional[np.ndarray],
              expert: ExpertFn, shared: Optional["tuple[np.ndarray, np.ndarray]"],
              spec: Spec, tokens: Optional[Sequence[int]] = None,
              force_idx: Optional[np.ndarray] = None):
    """h'_t = u_t + FFN_share(u_t) + sum over chosen r (ascending) of g_{r,t} FFN_r(u_t).

    x: [T, dim] float64.  expert(e) -> (W13_e [2I, dim], W2_e [dim, I]) float64.
    shared: (SW13 [2SI, dim], SW2 [dim, SI]) or None.  The gate runs on all T
    tokens; the output rows are computed for `tokens` (default all), in that
    order.  Returns (out [len(tokens), dim], GateResult).
    """
    x = np.asarray(x, np.float64)
    g = gate(x, w_gate, bias, spec, force_idx=force_idx)
    toks = np.arange(x.shape[0]) if tokens is None else np.asarray(tokens, dtype=np.int64)
    u = x[toks]
    routed = np.zeros_like(u)
    idx, w = g.idx[toks], g.w[toks]
    for e in np.unique(idx):               # ascending expert index, as the sum is ordered
        rows, slot = np.nonzero(idx == e)
        w13, w2 = expert(int(e))
        y = swiglu_ffn(u[rows], w13, w2)
        routed[rows] += w[rows, slot][:, None] * y
    out = routed
    if shared is not None:
        out = swiglu_ffn(u, shared[0], shared[1]) + out
    if spec.add_residual:
        out = u + out
    return out, g
