"""Seeded synthetic inputs for one MoE layer.

This module only draws random tensors and encodes them into their storage
formats (bf16, fp32, or fp8 e4m3 codes with one fp32 scale per 128x128 block).
It holds none of the layer's arithmetic: both the HIP path and the CPU oracle
receive exactly the tensors built here.

Recipe (the same for every shape):
  * x ~ N(0, 1), one row per token, stored in the activation dtype;
  * every weight matrix ~ N(0, 1/fan_in): fan_in = dim for the gate and for
    the gate/up projections, inter_dim for a routed down projection and
    n_shared*inter_dim for the shared down projection;
  * optional per-expert bias ~ U(-r, r), fp32;
  * optional skewed routing: gate rows scaled by c_e = (pi(e)+1)^-s for a
    seeded permutation pi, normalised to unit RMS, before rounding;
  * fp8: each 128x128 block of a weight matrix is stored as e4m3 codes q with
    scale s = max|W_block| / 448 (s = 1 for an all-zero block) and
    q = e4m3(W / s), round-to-nearest-even, clamped to +-448.

Values depend on the device the generator runs on (torch's CPU and GPU
generators differ); a test feeds the same tensors to both sides, so only
reproducibility per device matters.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import torch

from .configs import LayerShape

FP8_MAX = 448.0
FP8_BLOCK = 128

_TENSOR_IDS = {"x": 1, "w_gate": 2, "bias": 3, "w13": 4, "w2": 5,
               "sw13": 6, "sw2": 7, "zipf": 8, "dout": 9}

_TORCH_ACT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _gen(device, seed: int, tensor: str, sub: int = 0) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1_000_003 + _TENSOR_IDS[tensor] * 65_537 + sub) & 0x7FFF_FFFF_FFFF)
    return g


def _normal(shape, std, device, g) -> torch.Tensor:
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return t.mul_(std)


def quantize_e4m3_block128(w: torch.Tensor):
    """Encode a float32 [R, C] matrix as (e4m3 codes uint8 [R, C], scales fp32 [R/128, C/128])."""
    R, C = w.shape
    assert R % FP8_BLOCK == 0 and C % FP8_BLOCK == 0, (R, C)
    blk = w.reshape(R // FP8_BLOCK, FP8_BLOCK, C // FP8_BLOCK, FP8_BLOCK)
    amax = blk.abs().amax(dim=(1, 3))
    scale = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
    q = (blk / scale[:, None, :, None]).clamp_(-FP8_MAX, FP8_MAX)
    codes = q.reshape(R, C).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.contiguous(), scale.contiguous()


@dataclass
class LayerTensors:
    """Device tensors of one layer in their storage formats (see module doc)."""
    shape: LayerShape
    x: torch.Tensor                       # [T, dim] act dtype
    w_gate: torch.Tensor                  # [E, dim] act dtype
    bias: Optional[torch.Tensor]          # [E] fp32 or None
    w13: torch.Tensor                     # [E, 2I, dim]; rows [0,I) gate proj, [I,2I) up proj
    w2: torch.Tensor                      # [E, dim, I]
    sw13: Optional[torch.Tensor]          # [2*S*I, dim]; rows [0,S*I) gate, [S*I,2*S*I) up
    sw2: Optional[torch.Tensor]           # [dim, S*I]
    w13_scale: Optional[torch.Tensor] = None   # fp8: [E, 2I/128, dim/128]
    w2_scale: Optional[torch.Tensor] = None    # fp8: [E, dim/128, I/128]
    sw13_scale: Optional[torch.Tensor] = None  # fp8: [2SI/128, dim/128]
    sw2_scale: Optional[torch.Tensor] = None   # fp8: [dim/128, SI/128]
    extra: dict = field(default_factory=dict)


def _store_weight(w32: torch.Tensor, kind: str):
    if kind == "f32":
        return w32, None
    if kind == "bf16":
        return w32.to(torch.bfloat16), None
    if kind == "fp8":
        return quantize_e4m3_block128(w32)
    raise ValueError(kind)


def zipf_row_scale(shape: LayerShape, device) -> torch.Tensor:
    g = _gen("cpu", shape.seed, "zipf")
    perm = torch.randperm(shape.n_routed, generator=g)
    c = (perm.to(torch.float64) + 1.0) ** (-shape.zipf)
    c = c / torch.sqrt((c * c).mean())
    return c.to(torch.float32).to(device)


def make_x(shape: LayerShape, device, T: Optional[int] = None, seed_offset: int = 0) -> torch.Tensor:
    T = shape.T if T is None else T
    g = _gen(device, shape.seed + seed_offset, "x")
    return _normal((T, shape.dim), 1.0, device, g).to(_TORCH_ACT[shape.act])


def make_dout(shape: LayerShape, device="cpu", T: Optional[int] = None) -> torch.Tensor:
    """Upstream gradient dL/d(out) for the backward pass: N(0, 1), [T, dim] in the act dtype."""
    T = shape.T if T is None else T
    g = _gen(device, shape.seed, "dout")
    return _normal((T, shape.dim), 1.0, device, g).to(_TORCH_ACT[shape.act])


def make_gate_inputs(shape: LayerShape, device="cpu", T: Optional[int] = None):
    """(x, w_gate, bias) of one layer call: the same draws make_layer makes."""
    E, D = shape.n_routed, shape.dim
    act = _TORCH_ACT[shape.act]
    x = make_x(shape, device, T)

    wg = _normal((E, D), 1.0 / math.sqrt(D), device, _gen(device, shape.seed, "w_gate"))
    if shape.zipf is not None:
        wg.mul_(zipf_row_scale(shape, device)[:, None])
    w_gate = wg.to(act)

    bias = None
    if shape.bias_range is not None:
        g = _gen(device, shape.seed, "bias")
        bias = (torch.rand((E,), generator=g, device=device, dtype=torch.float32) * 2.0 - 1.0) * shape.bias_range
    return x, w_gate, bias


def make_layer(shape: LayerShape, device="cpu", T: Optional[int] = None,
               shared: bool = True) -> LayerTensors:
    """Draw every input of one layer call on `device` (x has T rows, default shape.T)."""
    E, D, I, S = shape.n_routed, shape.dim, shape.inter_dim, shape.n_shared
    x, w_gate, bias = make_gate_inputs(shape, device, T)

    w13_parts, w13_sc, w2_parts, w2_sc = [], [], [], []
    for e in range(E):
        a = _normal((2 * I, D), 1.0 / math.sqrt(D), device, _gen(device, shape.seed, "w13", e))
        q, s = _store_weight(a, shape.weight)
        w13_parts.append(q)
        w13_sc.append(s)
        del a
        b = _normal((D, I), 1.0 / math.sqrt(I), device, _gen(device, shape.seed, "w2", e))
        q, s = _store_weight(b, shape.weight)
        w2_parts.append(q)
        w2_sc.append(s)
        del b
    w13 = torch.stack(w13_parts)
    del w13_parts
    w2 = torch.stack(w2_parts)
    del w2_parts
    w13_scale = torch.stack(w13_sc) if shape.weight == "fp8" else None
    w2_scale = torch.stack(w2_sc) if shape.weight == "fp8" else None

    sw13 = sw2 = sw13_scale = sw2_scale = None
    if shared and S > 0:
        a = _normal((2 * S * I, D), 1.0 / math.sqrt(D), device, _gen(device, shape.seed, "sw13"))
        sw13, sw13_scale = _store_weight(a, shape.weight)
        del a
        b = _normal((D, S * I), 1.0 / math.sqrt(S * I), device, _gen(device, shape.seed, "sw2"))
        sw2, sw2_scale = _store_weight(b, shape.weight)
        del b

    return LayerTensors(shape=shape, x=x, w_gate=w_gate, bias=bias, w13=w13, w2=w2,
                        sw13=sw13, sw2=sw2, w13_scale=w13_scale, w2_scale=w2_scale,
                        sw13_scale=sw13_scale, sw2_scale=sw2_scale)
