"""ctypes binding of libmoe355.so: the C ABI's entry points under the same names.

Argument marshalling only: tensors become device pointers, the stream becomes
a hipStream_t, every status other than MOE_OK raises MoeError.  Every step of
the layer runs in the library's HIP kernels; there is no other implementation
to fall back on, and a missing library is an error.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

from .configs import LayerShape

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe355.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_DEVICE = range(5)
MOE_F32, MOE_BF16, MOE_FP8_E4M3_B128 = range(3)
MOE_SCORE_SIGMOID, MOE_SCORE_SOFTMAX = range(2)

_DTYPE = {"f32": MOE_F32, "bf16": MOE_BF16, "fp8": MOE_FP8_E4M3_B128}
_SCORE = {"sigmoid": MOE_SCORE_SIGMOID, "softmax": MOE_SCORE_SOFTMAX}


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


_STATUS_NAMES = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARG", 2: "MOE_ERR_UNSUPPORTED",
                 3: "MOE_ERR_WORKSPACE", 4: "MOE_ERR_DEVICE"}


class moe_config(ctypes.Structure):
    _fields_ = [("dim", ctypes.c_int32), ("n_routed", ctypes.c_int32), ("n_shared", ctypes.c_int32),
                ("n_groups", ctypes.c_int32), ("topk_groups", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("inter_dim", ctypes.c_int32), ("route_scale", ctypes.c_float),
                ("score_func", ctypes.c_int32), ("norm_topk", ctypes.c_int32),
                ("act_dtype", ctypes.c_int32), ("weight_dtype", ctypes.c_int32),
                ("add_residual", ctypes.c_int32), ("act_quant", ctypes.c_int32)]


class moe_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("w_gate", "bias", "w13", "w13_scale", "w2", "w2_scale", "sw13", "sw13_scale",
                 "sw2", "sw2_scale")]


class moe_routing(ctypes.Structure):
    _fields_ = [("tile_m", ctypes.c_int32), ("max_rows", ctypes.c_int32),
                ("max_tiles", ctypes.c_int32), ("pad_", ctypes.c_int32)] + \
               [(n, ctypes.c_void_p) for n in ("counts", "expert_off", "sorted_pair", "pair_row",
                                               "tile_expert", "tile_row", "n_tiles", "scratch",
                                               "act_q", "act_s")]


class moe_grads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("dx", "dw_gate", "dw13", "dw2", "dsw13", "dsw2")]


EXPORTED = ("moe_validate", "moe_routing_size", "moe_routing_init", "moe_workspace_size",
            "moe_status_str", "moe_last_error", "moe_gate", "moe_permute", "moe_expert_ffn",
            "moe_expert_up", "moe_expert_down", "moe_combine", "moe_forward", "moe_bias_update",
            "moe_quant_act", "moe_balance_loss", "moe_balance_loss_workspace_size",
            "moe_backward", "moe_backward_workspace_size", "moe_forward_static",
            "moe_expert_ffn_save", "moe_backward_saved")

_lib = None


def lib():
    """Load libmoe355.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m routed_expert_moe_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, I64, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    cfgp = ctypes.POINTER(moe_config)
    sig = {
        "moe_validate": [cfgp],
        "moe_routing_size": [cfgp, I64, ctypes.POINTER(SZ)],
        "moe_routing_init": [cfgp, I64, P, SZ, ctypes.POINTER(moe_routing)],
        "moe_workspace_size": [cfgp, I64, ctypes.POINTER(SZ)],
        "moe_gate": [cfgp, I64, P, P, P, P, P, P, P, P],
        "moe_permute": [cfgp, I64, P, ctypes.POINTER(moe_routing), P],
        "moe_expert_ffn": [cfgp, I64, P, ctypes.POINTER(moe_routing), ctypes.POINTER(moe_weights),
                           P, P, P, P, P],
        "moe_expert_up": [cfgp, I64, P, ctypes.POINTER(moe_routing), ctypes.POINTER(moe_weights),
                          P, P, P],
        "moe_expert_down": [cfgp, I64, ctypes.POINTER(moe_routing), ctypes.POINTER(moe_weights),
                            P, P, P, P, P],
        "moe_combine": [cfgp, I64, P, P, P, ctypes.POINTER(moe_routing), P, P, P],
        "moe_forward": [cfgp, I64, P, ctypes.POINTER(moe_weights), P, P, P, P, SZ, P],
        "moe_forward_static": [cfgp, I64, P, ctypes.POINTER(moe_weights), P, P, P, P],
        "moe_bias_update": [cfgp, I64, ctypes.POINTER(moe_routing), ctypes.c_float, P, P],
        "moe_quant_act": [cfgp, I64, P, ctypes.POINTER(moe_routing), P],
        "moe_balance_loss": [cfgp, I64, ctypes.c_int32, P, P, ctypes.c_float, P, ctypes.c_size_t, P, P],
        "moe_balance_loss_workspace_size": [cfgp, I64, ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)],
        "moe_backward_workspace_size": [cfgp, I64, ctypes.POINTER(SZ)],
        "moe_backward": [cfgp, I64, P, ctypes.POINTER(moe_weights), ctypes.POINTER(moe_routing), P, P, P,
                         P, P, ctypes.POINTER(moe_grads), P, SZ, P],
        "moe_expert_ffn_save": [cfgp, I64, P, ctypes.POINTER(moe_routing), ctypes.POINTER(moe_weights),
                                P, P, P, P, P, P, P],
        "moe_backward_saved": [cfgp, I64, P, ctypes.POINTER(moe_weights), ctypes.POINTER(moe_routing), P, P,
                               P, P, P, P, P, ctypes.POINTER(moe_grads), P, SZ, P],
    }
    for name, args in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    L.moe_status_str.argtypes = [ctypes.c_int]
    L.moe_status_str.restype = ctypes.c_char_p
    L.moe_last_error.argtypes = []
    L.moe_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(status: int):
    if status != MOE_OK:
        raise MoeError(status, lib().moe_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    return t.data_ptr()


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def _device_bytes(n: int, like: torch.Tensor) -> torch.Tensor:
    """A device byte buffer of at least n bytes on like's device (torch allocations are 256-byte aligned)."""
    return torch.empty(max(int(n), 256), dtype=torch.uint8, device=like.device)


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def config_of(shape: LayerShape) -> moe_config:
    return moe_config(dim=shape.dim, n_routed=shape.n_routed, n_shared=shape.n_shared,
                      n_groups=shape.n_groups, topk_groups=shape.topk_groups, top_k=shape.top_k,
                      inter_dim=shape.inter_dim, route_scale=shape.route_scale,
                      score_func=_SCORE[shape.score], norm_topk=shape.norm_topk,
                      act_dtype=_DTYPE[shape.act], weight_dtype=_DTYPE[shape.weight],
                      add_residual=shape.add_residual, act_quant=shape.act_quant)


def weights_of(layer) -> moe_weights:
    return moe_weights(w_gate=_ptr(layer.w_gate), bias=_ptr(layer.bias), w13=_ptr(layer.w13),
                       w13_scale=_ptr(layer.w13_scale), w2=_ptr(layer.w2), w2_scale=_ptr(layer.w2_scale),
                       sw13=_ptr(layer.sw13), sw13_scale=_ptr(layer.sw13_scale), sw2=_ptr(layer.sw2),
                       sw2_scale=_ptr(layer.sw2_scale))


# ---- host-only queries --------------------------------------------------------
def moe_validate(cfg: moe_config) -> None:
    _check(lib().moe_validate(ctypes.byref(cfg)))


def moe_routing_size(cfg: moe_config, T: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().moe_routing_size(ctypes.byref(cfg), T, ctypes.byref(n)))
    return n.value


def moe_workspace_size(cfg: moe_config, T: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().moe_workspace_size(ctypes.byref(cfg), T, ctypes.byref(n)))
    return n.value


def moe_routing_init(cfg: moe_config, T: int, buf_ptr: int, nbytes: int) -> moe_routing:
    r = moe_routing()
    _check(lib().moe_routing_init(ctypes.byref(cfg), T, buf_ptr, nbytes, ctypes.byref(r)))
    return r


@dataclass
class Routing:
    """A routing buffer on the device plus int32 views of its arrays."""
    struct: moe_routing
    buf: torch.Tensor
    counts: torch.Tensor
    expert_off: torch.Tensor
    sorted_pair: torch.Tensor
    pair_row: torch.Tensor
    tile_expert: torch.Tensor
    tile_row: torch.Tensor
    n_tiles: torch.Tensor
    act_q: Optional[torch.Tensor] = None     # act_quant: [T, D] e4m3 codes (uint8)
    act_s: Optional[torch.Tensor] = None     # act_quant: [T, D/128] fp32 scales


def make_routing(cfg: moe_config, T: int, device="cuda") -> Routing:
    nbytes = moe_routing_size(cfg, T)
    buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
    r = moe_routing_init(cfg, T, buf.data_ptr(), buf.numel())
    base = buf.data_ptr()

    def view(ptr, n):
        off = ptr - base
        return buf[off: off + 4 * n].view(torch.int32)
    P = T * cfg.top_k
    act_q = act_s = None
    if cfg.act_quant and T > 0:
        nb = cfg.dim // 128
        act_q = buf[r.act_q - base: r.act_q - base + T * cfg.dim].view(T, cfg.dim)
        act_s = buf[r.act_s - base: r.act_s - base + 4 * T * nb].view(torch.float32).view(T, nb)
    return Routing(r, buf, view(r.counts, cfg.n_routed), view(r.expert_off, cfg.n_routed + 1),
                   view(r.sorted_pair, r.max_rows), view(r.pair_row, P),
                   view(r.tile_expert, r.max_tiles), view(r.tile_row, r.max_tiles), view(r.n_tiles, 1),
                   act_q, act_s)


# ---- the forward pass, step by step ---------------------------------------------
def moe_gate(cfg: moe_config, T: int, x, w_gate, bias, logits, topk_idx, topk_w, keys=None,
             stream=None) -> None:
    _check(lib().moe_gate(ctypes.byref(cfg), T, _ptr(x), _ptr(w_gate), _ptr(bias), _ptr(logits),
                          _ptr(topk_idx), _ptr(topk_w), _ptr(keys), _stream(stream)))


def moe_permute(cfg: moe_config, T: int, topk_idx, routing: Routing, stream=None) -> None:
    _check(lib().moe_permute(ctypes.byref(cfg), T, _ptr(topk_idx), ctypes.byref(routing.struct),
                             _stream(stream)))


def moe_expert_ffn(cfg: moe_config, T: int, x, routing: Routing, weights: moe_weights, h, y_pairs,
                   hs=None, z=None, stream=None) -> None:
    _check(lib().moe_expert_ffn(ctypes.byref(cfg), T, _ptr(x), ctypes.byref(routing.struct),
                                ctypes.byref(weights), _ptr(h), _ptr(y_pairs), _ptr(hs), _ptr(z),
                                _stream(stream)))


def moe_expert_ffn_save(cfg: moe_config, T: int, x, routing: Routing, weights: moe_weights, h, y_pairs,
                        hs, z, ab, abs_, stream=None) -> None:
    """moe_expert_ffn that also keeps the gate/up pre-activations: ab [max_rows, 2I] and
    abs_ [T, 2SI] (None without a shared expert), fp32."""
    _check(lib().moe_expert_ffn_save(ctypes.byref(cfg), T, _ptr(x), ctypes.byref(routing.struct),
                                     ctypes.byref(weights), _ptr(h), _ptr(y_pairs), _ptr(hs), _ptr(z),
                                     _ptr(ab), _ptr(abs_), _stream(stream)))


def moe_expert_up(cfg: moe_config, T: int, x, routing: Routing, weights: moe_weights, h, hs=None,
                  stream=None) -> None:
    _check(lib().moe_expert_up(ctypes.byref(cfg), T, _ptr(x), ctypes.byref(routing.struct),
                               ctypes.byref(weights), _ptr(h), _ptr(hs), _stream(stream)))


def moe_expert_down(cfg: moe_config, T: int, routing: Routing, weights: moe_weights, h, hs, y_pairs,
                    z=None, stream=None) -> None:
    _check(lib().moe_expert_down(ctypes.byref(cfg), T, ctypes.byref(routing.struct),
                                 ctypes.byref(weights), _ptr(h), _ptr(hs), _ptr(y_pairs), _ptr(z),
                                 _stream(stream)))


def moe_combine(cfg: moe_config, T: int, u, z, y_pairs, routing: Routing, topk_w, out,
                stream=None) -> None:
    _check(lib().moe_combine(ctypes.byref(cfg), T, _ptr(u), _ptr(z), _ptr(y_pairs),
                             ctypes.byref(routing.struct), _ptr(topk_w), _ptr(out), _stream(stream)))


def moe_quant_act(cfg: moe_config, T: int, x, routing: Routing, stream=None) -> None:
    _check(lib().moe_quant_act(ctypes.byref(cfg), T, _ptr(x), ctypes.byref(routing.struct), _stream(stream)))


def moe_balance_loss_workspace_size(cfg: moe_config, T: int, seq_len: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().moe_balance_loss_workspace_size(ctypes.byref(cfg), T, int(seq_len), ctypes.byref(n)))
    return n.value


def moe_balance_loss(cfg: moe_config, T: int, seq_len: int, logits, topk_idx, alpha: float, loss,
                     stream=None, workspace=None) -> None:
    """workspace: a device buffer of >= moe_balance_loss_workspace_size bytes (allocated here if None)."""
    if workspace is None:
        workspace = _device_bytes(moe_balance_loss_workspace_size(cfg, T, seq_len), logits)
    _check(lib().moe_balance_loss(ctypes.byref(cfg), T, int(seq_len), _ptr(logits), _ptr(topk_idx),
                                  float(alpha), _ptr(workspace), _nbytes(workspace), _ptr(loss),
                                  _stream(stream)))


def moe_backward_workspace_size(cfg: moe_config, T: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().moe_backward_workspace_size(ctypes.byref(cfg), T, ctypes.byref(n)))
    return n.value


@dataclass
class Grads:
    """Gradient buffers of moe_backward (device tensors)."""
    dx: torch.Tensor         # [T, D] act dtype
    dw_gate: torch.Tensor    # [E, D] fp32
    dw13: torch.Tensor       # [E, 2I, D] fp32
    dw2: torch.Tensor        # [E, D, I] fp32
    dsw13: Optional[torch.Tensor] = None   # [2SI, D] fp32
    dsw2: Optional[torch.Tensor] = None    # [D, SI] fp32

    @staticmethod
    def empty(cfg: moe_config, T: int, act_dtype, device="cuda") -> "Grads":
        D, E, I, SI = cfg.dim, cfg.n_routed, cfg.inter_dim, cfg.n_shared * cfg.inter_dim
        f = dict(dtype=torch.float32, device=device)
        return Grads(torch.empty(T, D, dtype=act_dtype, device=device), torch.empty(E, D, **f),
                     torch.empty(E, 2 * I, D, **f), torch.empty(E, D, I, **f),
                     torch.empty(2 * SI, D, **f) if SI else None, torch.empty(D, SI, **f) if SI else None)

    def struct(self) -> moe_grads:
        return moe_grads(*(_ptr(t) for t in (self.dx, self.dw_gate, self.dw13, self.dw2, self.dsw13, self.dsw2)))


def moe_backward(cfg: moe_config, T: int, x, weights: moe_weights, routing: Routing, topk_idx, topk_w,
                 logits, y_pairs, dout, grads: Grads, workspace=None, stream=None) -> None:
    """workspace: a device buffer of >= moe_backward_workspace_size bytes (allocated here if None)."""
    if workspace is None:
        workspace = _device_bytes(moe_backward_workspace_size(cfg, T), x)
    g = grads.struct()
    _check(lib().moe_backward(ctypes.byref(cfg), T, _ptr(x), ctypes.byref(weights), ctypes.byref(routing.struct),
                              _ptr(topk_idx), _ptr(topk_w), _ptr(logits), _ptr(y_pairs), _ptr(dout),
                              ctypes.byref(g), _ptr(workspace), _nbytes(workspace), _stream(stream)))


def moe_backward_saved(cfg: moe_config, T: int, x, weights: moe_weights, routing: Routing, topk_idx, topk_w,
                       logits, y_pairs, dout, ab, abs_, grads: Grads, workspace=None, stream=None) -> None:
    """moe_backward reading the pre-activations moe_expert_ffn_save kept (ab, abs_)."""
    if workspace is None:
        workspace = _device_bytes(moe_backward_workspace_size(cfg, T), x)
    g = grads.struct()
    _check(lib().moe_backward_saved(ctypes.byref(cfg), T, _ptr(x), ctypes.byref(weights),
                                    ctypes.byref(routing.struct), _ptr(topk_idx), _ptr(topk_w), _ptr(logits),
                                    _ptr(y_pairs), _ptr(dout), _ptr(ab), _ptr(abs_), ctypes.byref(g),
                                    _ptr(workspace), _nbytes(workspace), _stream(stream)))


def moe_bias_update(cfg: moe_config, T: int, routing: Routing, gamma: float, bias, stream=None) -> None:
    _check(lib().moe_bias_update(ctypes.byref(cfg), T, ctypes.byref(routing.struct), float(gamma),
                                 _ptr(bias), _stream(stream)))


def moe_forward(cfg: moe_config, T: int, x, weights: moe_weights, out, topk_idx=None, topk_w=None,
                ws: torch.Tensor = None, stream=None) -> None:
    _check(lib().moe_forward(ctypes.byref(cfg), T, _ptr(x), ctypes.byref(weights), _ptr(out),
                             _ptr(topk_idx), _ptr(topk_w), _ptr(ws), 0 if ws is None else ws.numel(),
                             _stream(stream)))


def moe_forward_static(cfg: moe_config, T: int, x, weights: moe_weights, out, topk_idx=None, topk_w=None,
                       stream=None) -> None:
    _check(lib().moe_forward_static(ctypes.byref(cfg), T, _ptr(x), ctypes.byref(weights), _ptr(out),
                                    _ptr(topk_idx), _ptr(topk_w), _stream(stream)))


# ---- convenience: one layer's state on the device ----------------------------------
class MoELayer:
    """Holds a layer's config, weights and workspace; runs moe_forward."""

    def __init__(self, layer, T_max: Optional[int] = None):
        self.layer = layer
        self.shape = layer.shape
        self.cfg = config_of(layer.shape)
        moe_validate(self.cfg)
        self.weights = weights_of(layer)
        self.T_max = layer.x.shape[0] if T_max is None else T_max
        self.ws = torch.empty(max(moe_workspace_size(self.cfg, self.T_max), 256), dtype=torch.uint8,
                              device=layer.x.device)

    def forward(self, x: torch.Tensor, out: Optional[torch.Tensor] = None, topk_idx=None,
                topk_w=None, stream=None) -> torch.Tensor:
        T = x.shape[0]
        if T > self.T_max:
            raise ValueError(f"T={T} exceeds the workspace's T_max={self.T_max}")
        if out is None:
            out = torch.empty_like(x)
        moe_forward(self.cfg, T, x, self.weights, out, topk_idx, topk_w, self.ws, stream)
        return out
