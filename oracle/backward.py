"""Oracle: the backward pass of one DeepSeekMoE layer, in plain float64 NumPy.

TEST INFRASTRUCTURE.  Only the tests, the smoke check of the package entry file
and the CPU-baseline leg of the benchmark may import this module.  The library
never imports it and shares no code with it.

What is computed
----------------
The pages define the forward pass only (DeepSeek-V3 notes page: the layer
output h'_t = u_t + FFN_share(u_t) + sum_r g_{r,t} FFN_r(u_t), the gate flow in
five steps, the auxiliary-loss-free bias that steers selection only).  The
backward pass is the gradient of a scalar loss L = sum_t <dout_t, h'_t> with
respect to everything the forward pass is differentiable in: the tokens u, the
gate matrix W_g, every routed expert's W1/W3/W2 and the shared expert's.  It is
the chain rule applied to the forward steps in reverse order, written out:

  * combine:  dw_{t,k} = <dout_t, FFN_{e(t,k)}(u_t)>,   dy_{t,k} = w_{t,k} dout_t;
              the residual passes dout_t to du_t, the shared expert gets dout_t.
  * SwiGLU expert y = W2 h, h = silu(a) * c, a = W1 u, c = W3 u:
              dW2 = dy^T h,  dh = dy W2,  da = dh * c * silu'(a),  dc = dh * silu(a),
              dW1 = da^T u,  dW3 = dc^T u,  du = da W1 + dc W3,
              silu'(a) = sigmoid(a) (1 + a (1 - sigmoid(a))).
  * route weights w_k = route_scale * s_{e_k} / S (S = sum of the chosen s) when
    renormalised, else route_scale * s_{e_k}:
              ds_{e_j} = rs * (dw_j / S - sum_k dw_k s_{e_k} / S^2)   (renormalised)
              ds_{e_j} = rs * dw_j                                    (plain),
    zero for experts that were not chosen.  The selection itself (top-k over
    s + b, group masking) is piecewise constant: no gradient flows through it,
    so the bias b gets none.
  * scores:   sigmoid  dl = ds * s (1 - s);
              softmax  dl = s * (ds - sum_e ds_e s_e)   (over all experts).
  * gate:     du += dl W_g,   dW_g = dl^T u.

Readings (also in the design notes): the loss is linear in the output (any
upstream gradient dout); gradients are exact float64 values of the forward
oracle's own function (same SwiGLU reading, same W13 = [W1; W3] stacking, the
S shared experts as one SwiGLU of hidden S*I).

Pinned by tests/test_backward_pins.py against central finite differences of
the forward oracle (oracle/moe_oracle.py) and against invariants of the
formulas (scale invariance of renormalised weights, shift invariance of the
softmax).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np

from .moe_oracle import GateResult, Spec, gate, sigmoid, swiglu_ffn


def swiglu_ffn_backward(xr: np.ndarray, w13: np.ndarray, w2: np.ndarray, dy: np.ndarray):
    """Gradients of y = W2 (silu(W1 u) * (W3 u)) row by row, given dL/dy.

    Returns (du [rows, dim], dW13 [2I, dim], dW2 [dim, I])."""
    inter = w13.shape[0] // 2
    w1, w3 = w13[:inter], w13[inter:]
    a = xr @ w1.T
    c = xr @ w3.T
    sa = sigmoid(a)
    h = a * sa * c
    dw2 = dy.T @ h
    dh = dy @ w2
    da = dh * c * (sa * (1.0 + a * (1.0 - sa)))
    dc = dh * a * sa
    dw13 = np.concatenate([da.T @ xr, dc.T @ xr], axis=0)
    du = da @ w1 + dc @ w3
    return du, dw13, dw2


def route_weights_backward(s: np.ndarray, idx: np.ndarray, dw: np.ndarray, spec: Spec) -> np.ndarray:
    """dL/ds [T, E] from dL/dw [T, K] through gather, optional renormalisation and route_scale."""
    dwr = np.asarray(dw, np.float64) * spec.route_scale
    sel = np.take_along_axis(s, idx, axis=-1)
    if spec.normalise:
        tot = sel.sum(axis=-1, keepdims=True)
        dsel = dwr / tot - (dwr * sel).sum(axis=-1, keepdims=True) / (tot * tot)
    else:
        dsel = dwr
    ds = np.zeros_like(s)
    np.put_along_axis(ds, idx, dsel, axis=-1)    # the K chosen experts of a token are distinct
    return ds


def gate_scores_backward(s: np.ndarray, ds: np.ndarray, score: str) -> np.ndarray:
    """dL/dlogits from dL/ds: sigmoid elementwise, softmax over each token's experts."""
    if score == "sigmoid":
        return ds * s * (1.0 - s)
    if score == "softmax":
        return s * (ds - (ds * s).sum(axis=-1, keepdims=True))
    raise ValueError(score)


@dataclass
class LayerGrads:
    dx: np.ndarray                      # [T, dim]
    dw_gate: np.ndarray                 # [E, dim]
    dw13: Dict[int, np.ndarray]         # expert -> [2I, dim] (only experts that were chosen)
    dw2: Dict[int, np.ndarray]          # expert -> [dim, I]
    dsw13: Optional[np.ndarray]         # [2SI, dim]
    dsw2: Optional[np.ndarray]          # [dim, SI]
    dw: np.ndarray                      # [T, K] dL/d(route weight)
    dlogits: np.ndarray                 # [T, E]
    gate: GateResult = field(repr=False)


def moe_layer_backward(x: np.ndarray, w_gate: np.ndarray, bias: Optional[np.ndarray], expert,
                       shared, spec: Spec, dout: np.ndarray,
                       force_idx: Optional[np.ndarray] = None) -> LayerGrads:
    """Gradients of L = sum_t <dout_t, h'_t> for the layer of moe_oracle.moe_layer.

    Arguments as moe_layer (expert(e) -> (W13_e, W2_e) float64; shared = (SW13, SW2)
    or None); dout [T, dim].  `force_idx` fixes the selection, as in the forward."""
    x = np.asarray(x, np.float64)
    w_gate = np.asarray(w_gate, np.float64)
    dout = np.asarray(dout, np.float64)
    g = gate(x, w_gate, bias, spec, force_idx=force_idx)
    T, K = g.idx.shape
    dx = dout.copy() if spec.add_residual else np.zeros_like(x)

    dsw13 = dsw2 = None
    if shared is not None:
        dxs, dsw13, dsw2 = swiglu_ffn_backward(x, shared[0], shared[1], dout)
        dx += dxs

    dw = np.zeros((T, K))
    dw13, dw2 = {}, {}
    for e in np.unique(g.idx):
        rows, slot = np.nonzero(g.idx == e)       # each token lists e at most once
        w13, w2 = expert(int(e))
        y = swiglu_ffn(x[rows], w13, w2)
        dw[rows, slot] = (dout[rows] * y).sum(axis=-1)
        dy = g.w[rows, slot][:, None] * dout[rows]
        dxr, dw13[int(e)], dw2[int(e)] = swiglu_ffn_backward(x[rows], w13, w2, dy)
        dx[rows] += dxr

    ds = route_weights_backward(g.s, g.idx, dw, spec)
    dl = gate_scores_backward(g.s, ds, spec.score)
    dx += dl @ w_gate
    dw_gate = dl.T @ x
    return LayerGrads(dx, dw_gate, dw13, dw2, dsw13, dsw2, dw, dl, g)
