"""Helpers for the GPU parity tests: run the library's steps and compare with
the oracle under the index-certification protocol.

Index parity protocol.  The GPU ranks fp32 keys; the oracle ranks float64
keys.  (1) Replaying the oracle's selection on the GPU's own exported fp32
keys must give the GPU's experts exactly, for every token: this pins group
scoring, masking, top-k and tie-breaks.  (2) With eps = max |key_gpu -
key_oracle|, a token whose oracle selection gaps exceed 4*eps cannot change
its selection under that perturbation; on such certified tokens the GPU's
experts must equal the oracle's exactly.  Uncertified tokens are counted and
their values are checked against the oracle run on the GPU's selection.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from routed_expert_moe_amd import binding as B
from oracle_bridge import bias_f64, spec_of, to_f64

TOL = {"f32": 1e-5, "bf16": 2e-2, "fp8": 6e-2}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_gate(layer, x=None):
    cfg = B.config_of(layer.shape)
    x = layer.x if x is None else x
    T, E, K = x.shape[0], layer.shape.n_routed, layer.shape.top_k
    dev = x.device
    logits = torch.empty(T, E, dtype=torch.float32, device=dev)
    keys = torch.empty(T, E, dtype=torch.float32, device=dev)
    idx = torch.empty(T, K, dtype=torch.int32, device=dev)
    w = torch.empty(T, K, dtype=torch.float32, device=dev)
    B.moe_gate(cfg, T, x, layer.w_gate, layer.bias, logits, idx, w, keys)
    torch.cuda.synchronize()
    return (logits.cpu().numpy(), keys.cpu().numpy(), idx.cpu().numpy().astype(np.int64),
            w.cpu().numpy())


def certify(layer, idx_gpu, keys_gpu, g_ref):
    """Returns (certified mask, eps).  Asserts protocol parts (1) and (2)."""
    spec = spec_of(layer.shape)
    has_bias = layer.bias is not None
    replay = oracle.select_experts(keys_gpu.astype(np.float32), spec, has_bias)
    bad = np.nonzero((replay != idx_gpu).any(axis=1))[0]
    assert bad.size == 0, f"GPU selection differs from its own keys on tokens {bad[:10]}"
    eps = float(np.max(np.abs(keys_gpu.astype(np.float64) - g_ref.key)))
    cert = (g_ref.expert_gap > 4 * eps) & (g_ref.group_gap > 4 * eps)
    mism = np.nonzero(cert & (idx_gpu != g_ref.idx).any(axis=1))[0]
    assert mism.size == 0, f"certified tokens {mism[:10]} chose other experts (eps={eps:.3g})"
    return cert, eps


def rel_err(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-30))
