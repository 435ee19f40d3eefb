"""GPU parity of the gate logits GEMM's tile edges against the float64 oracle.

moe_gate forms logits = x W_g^T (DeepSeek-V3 notes page, gate flow, step 1) on
tiles of 64 tokens by 64 or 128 experts.  These shapes put the edges of that
tiling under test: a ragged last row tile, a partly filled last column block,
an expert count that is not a multiple of four (column-by-column stores), more
than 256 experts, a logits buffer that is only 4-byte aligned, and a model
width that is not a multiple of 128 (handled by the other GEMM).  The
logits must match the oracle's to 1e-5 of their largest magnitude (fp32
accumulation of exact bf16 products), and the selection must pass the
certification protocol of tests/parity.py.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle_bridge import bias_f64, spec_of, to_f64
from parity import certify, rel_err, say
from routed_expert_moe_amd import binding as B
from routed_expert_moe_amd import synth
from routed_expert_moe_amd.configs import LayerShape

pytestmark = pytest.mark.gpu


def _shape(name, T, D, E, groups, keep, K, score="sigmoid", seed=41):
    return LayerShape(name=name, T=T, dim=D, n_routed=E, n_groups=groups, topk_groups=keep, top_k=K,
                      n_shared=0, inter_dim=64, score=score, route_scale=2.5 if score == "sigmoid" else 1.0,
                      act="bf16", weight="bf16", seed=seed, bias_range=0.05 if score == "sigmoid" else None)


SHAPES = {
    # 90 experts: one full 64-wide block and one of 26 columns, scalar stores
    "E90_T200": _shape("gate_E90_T200", T=200, D=256, E=90, groups=1, keep=1, K=6, score="softmax"),
    # 320 experts: 128-wide blocks, the last half filled; 65 tokens: one row of the second row tile
    "E320_T65": _shape("gate_E320_T65", T=65, D=512, E=320, groups=8, keep=4, K=8),
    # 256 experts at a long K, T = 64 exactly (one row tile, the smallest T on this path)
    "E256_T64_D7168": _shape("gate_E256_T64", T=64, D=7168, E=256, groups=8, keep=4, K=8),
    # 160 experts (three 64-wide blocks, the last of 32), 1000 tokens
    "E160_T1000": _shape("gate_E160_T1000", T=1000, D=1024, E=160, groups=1, keep=1, K=6, score="softmax"),
    # a model width that is not a multiple of 128: the 128 x 128 register-staged tiles instead
    "E64_D320_T100": _shape("gate_E64_D320", T=100, D=320, E=64, groups=4, keep=2, K=6),
}


class _Layer:
    def __init__(self, shape):
        self.shape = shape
        self.x, self.w_gate, self.bias = synth.make_gate_inputs(shape, device="cuda")


def _gate(layer, logits_offset=0):
    sh = layer.shape
    T, E, K = sh.T, sh.n_routed, sh.top_k
    cfg = B.config_of(sh)
    buf = torch.full((T * E + logits_offset,), float("nan"), dtype=torch.float32, device="cuda")
    logits = buf[logits_offset:].view(T, E)
    keys = torch.empty(T, E, dtype=torch.float32, device="cuda")
    idx = torch.empty(T, K, dtype=torch.int32, device="cuda")
    w = torch.empty(T, K, dtype=torch.float32, device="cuda")
    B.moe_gate(cfg, T, layer.x, layer.w_gate, layer.bias, logits, idx, w, keys)
    torch.cuda.synchronize()
    return (buf.cpu().numpy(), logits.cpu().numpy(), keys.cpu().numpy(),
            idx.cpu().numpy().astype(np.int64), w.cpu().numpy())


def _check(layer, logits_offset=0):
    sh = layer.shape
    buf, logits, keys, idx, w = _gate(layer, logits_offset)
    g = oracle.gate(to_f64(layer.x), to_f64(layer.w_gate), bias_f64(layer), spec_of(sh))
    err = rel_err(logits, g.logits)
    say(f"[gate] {sh.name} offset={logits_offset} logits rel err {err:.3g}")
    assert np.isfinite(logits).all()
    assert err < 1e-5
    assert np.isnan(buf[:logits_offset]).all()      # nothing written before the logits
    cert, eps = certify(layer, idx, keys, g)
    assert (~cert).mean() < 0.02
    assert np.max(np.abs(w[cert] - g.w[cert])) <= 1e-5 * sh.route_scale


@pytest.mark.parametrize("name", list(SHAPES))
def test_gate_logits_tile_edges(name):
    _check(_Layer(SHAPES[name]))


def test_gate_logits_unaligned_output():
    # logits one float past a 16-byte boundary: the kernel must fall back to 4-byte stores
    _check(_Layer(SHAPES["E256_T64_D7168"].with_(name="gate_E256_unaligned", T=130)), logits_offset=1)
