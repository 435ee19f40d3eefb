"""Oracle: the auxiliary-loss-free bias update of DeepSeekMoE routing.

TEST INFRASTRUCTURE.  Only the tests, the smoke check of the package entry file
and the CPU-baseline leg of the benchmark may import this module.  The library
never imports it and shares no code with it.

What is computed, and where the pages state it
----------------------------------------------
  * DeepSeek-V3 notes page (73biji.xyz/llm_pp_dsv3), "V3 improvement 1": the
    ranked quantity is s_{i,t} + b_i, and b_i is adjusted as training runs
    according to each expert's load, at a speed set by gamma.
  * DeepSeek-R1 analysis page (deepseek.csdn.net), MoE hyper-parameters
    paragraph: the routing adds no balance loss term; each expert's call
    frequency is monitored, an overloaded expert's bias is lowered and an
    underloaded expert's bias is raised, at a rate given by a hyper-parameter.

Readings where the pages are silent (also listed in the design notes):
  * the load of expert e is the number of (token, slot) pairs of the batch
    routed to it; the balanced load is the mean T*K/E;
  * "overloaded" means load > mean, "underloaded" load < mean; an expert at
    exactly the mean keeps its bias; the comparison is exact (load*E vs T*K in
    integers);
  * the step is b_e <- b_e - gamma (overloaded) or b_e + gamma (underloaded),
    one float32 addition on the float32 bias (the bias is stored in float32;
    the pages fix no other precision).
"""
from __future__ import annotations

import numpy as np


def expert_loads(idx: np.ndarray, n_routed: int) -> np.ndarray:
    """Pairs routed to each expert: how often the batch called it (R1 analysis page)."""
    idx = np.asarray(idx).ravel()
    return np.bincount(idx[(idx >= 0) & (idx < n_routed)], minlength=n_routed).astype(np.int64)


def bias_update(bias: np.ndarray, loads: np.ndarray, n_tokens: int, top_k: int,
                gamma: float) -> np.ndarray:
    """One balancing step: lower the bias of overloaded experts, raise underloaded ones.

    DeepSeek-V3 notes page, "V3 improvement 1" (b_i follows the load, speed gamma);
    R1 analysis page, MoE hyper-parameters paragraph (overloaded -> lower,
    underloaded -> raise).  Returns a new float32 array.
    """
    b = np.array(bias, dtype=np.float32, copy=True)
    E = b.shape[0]
    g = np.float32(gamma)
    total = int(n_tokens) * int(top_k)          # sum of all loads; the mean is total / E
    for e in range(E):
        scaled = int(loads[e]) * E               # load_e > total / E  <=>  load_e * E > total
        if scaled > total:
            b[e] = b[e] - g
        elif scaled < total:
            b[e] = b[e] + g
    return b


def sequence_balance_loss(logits: np.ndarray, idx: np.ndarray, score: str, alpha: float,
                          seq_len: int) -> np.ndarray:
    """Sequence-wise balance loss, one value per sequence of seq_len tokens.

    DeepSeek-V3 notes page, "V3 improvement 2" (the paper's eqs. 17-20):
        L_Bal = alpha * sum_i f_i * P_i,
        f_i = E / (K * T_s) * #{t : i is among token t's chosen experts},
        s'_{i,t} = s_{i,t} / sum_j s_{j,t},   P_i = (1/T_s) * sum_t s'_{i,t},
    over the T_s = seq_len tokens of a sequence.  s is the unbiased score of
    the gate (sigmoid of the logit, or the softmax probability); the chosen
    experts are the routing the layer used (idx).  float64 throughout.
    """
    l = np.asarray(logits, np.float64)
    T, E = l.shape
    K = idx.shape[1]
    assert T % seq_len == 0, (T, seq_len)
    if score == "sigmoid":
        s = 1.0 / (1.0 + np.exp(-l))
    else:
        z = np.exp(l - l.max(axis=1, keepdims=True))
        s = z / z.sum(axis=1, keepdims=True)
    sn = s / s.sum(axis=1, keepdims=True)
    out = np.empty(T // seq_len)
    for q in range(T // seq_len):
        rows = slice(q * seq_len, (q + 1) * seq_len)
        counts = expert_loads(idx[rows], E).astype(np.float64)
        f = counts * E / (K * seq_len)
        P = sn[rows].mean(axis=0)
        out[q] = alpha * float(np.dot(f, P))
    return out
