"""Test glue: hand the generator's tensors to the CPU oracle.

Converts torch storage (fp32, bf16 bit patterns, fp8 codes + block scales) into
the oracle's float64 inputs through the oracle's own decoders, and maps a
LayerShape onto the oracle's Spec.  Nothing here computes the layer.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from oracle import w8a8
from routed_expert_moe_amd.configs import LayerShape


def spec_of(shape: LayerShape) -> oracle.Spec:
    return oracle.Spec(n_routed=shape.n_routed, n_groups=shape.n_groups,
                       topk_groups=shape.topk_groups, top_k=shape.top_k, score=shape.score,
                       route_scale=shape.route_scale, norm_topk=shape.norm_topk,
                       add_residual=shape.add_residual)


def to_f64(t: torch.Tensor) -> np.ndarray:
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.float32:
        return t.numpy().astype(np.float64)
    if t.dtype == torch.bfloat16:
        return oracle.decode_bf16(t.view(torch.int16).numpy().view(np.uint16))
    raise TypeError(t.dtype)


def weight_f64(q: torch.Tensor, scale, kind: str) -> np.ndarray:
    if kind == "fp8":
        return oracle.dequant_e4m3_block128(q.detach().cpu().numpy(), scale.detach().cpu().numpy())
    return to_f64(q)


def weight_f64_torch(q: torch.Tensor, scale, kind: str) -> np.ndarray:
    """The same exact float64 values as weight_f64, converted by torch where the tensor lives.

    Every stored value (bf16, fp32, e4m3 code times its fp32 block scale) is exact
    in float64, so only the speed differs (the benchmark's timing of the oracle
    excludes weight decoding and uses this to keep its own run short)."""
    if kind == "fp8":
        v = q.view(torch.float8_e4m3fn).to(torch.float64)
        R, C = v.shape
        s = scale.to(torch.float64)
        v = (v.view(R // 128, 128, C // 128, 128) * s[:, None, :, None]).view(R, C)
        return v.cpu().numpy()
    return q.to(torch.float64).cpu().numpy()


def expert_fn(layer, fast: bool = False):
    kind = layer.shape.weight
    conv = weight_f64_torch if fast else weight_f64

    def get(e: int):
        s13 = layer.w13_scale[e] if kind == "fp8" else None
        s2 = layer.w2_scale[e] if kind == "fp8" else None
        return conv(layer.w13[e], s13, kind), conv(layer.w2[e], s2, kind)
    return get


def shared_pair(layer):
    if layer.sw13 is None:
        return None
    kind = layer.shape.weight
    return (weight_f64(layer.sw13, layer.sw13_scale, kind),
            weight_f64(layer.sw2, layer.sw2_scale, kind))


def bias_f64(layer):
    return None if layer.bias is None else layer.bias.detach().cpu().numpy().astype(np.float64)


def run_oracle(layer, tokens=None, force_idx=None, x=None, fast=False):
    """Oracle forward of `layer` (optionally on another x and a token subset);
    the fp8 W8A8 layer when the shape quantises its activations.  fast: expert
    weights converted to float64 by torch (the same exact values, quicker at
    full size)."""
    xx = to_f64(layer.x if x is None else x)
    fn = w8a8.moe_layer_w8a8 if layer.shape.act_quant else oracle.moe_layer
    return fn(xx, to_f64(layer.w_gate), bias_f64(layer), expert_fn(layer, fast=fast), shared_pair(layer),
              spec_of(layer.shape), tokens=tokens, force_idx=force_idx)
