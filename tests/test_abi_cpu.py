"""The C ABI on the CPU: the library loads, exports every entry point its
header declares, and validates arguments on the host before any launch (so
every error path here runs without a GPU)."""
import ctypes
import os
import re

import pytest

from routed_expert_moe_amd import binding as B
from routed_expert_moe_amd import configs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe355.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = B.lib()
    names = _declared()
    assert set(names) >= {"moe_gate", "moe_permute", "moe_expert_ffn", "moe_combine", "moe_forward"}
    for n in names:
        assert hasattr(L, n), n
    assert set(B.EXPORTED) == set(names)


def test_struct_sizes_match_header_layout():
    assert ctypes.sizeof(B.moe_config) == 14 * 4
    assert ctypes.sizeof(B.moe_weights) == 10 * 8
    assert ctypes.sizeof(B.moe_routing) == 16 + 10 * 8


@pytest.mark.parametrize("shape", configs.ALL, ids=lambda s: s.name)
def test_named_shapes_validate(shape):
    B.moe_validate(B.config_of(shape))
    assert B.moe_workspace_size(B.config_of(shape), shape.T) > 0
    assert B.moe_routing_size(B.config_of(shape), shape.T) > 0


def _cfg(**kw):
    c = B.config_of(configs.TINY_F32)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


@pytest.mark.parametrize("kw,status", [
    (dict(n_groups=3), B.MOE_ERR_INVALID_ARG),            # 16 % 3 != 0
    (dict(topk_groups=0), B.MOE_ERR_INVALID_ARG),
    (dict(topk_groups=5), B.MOE_ERR_INVALID_ARG),
    (dict(top_k=9), B.MOE_ERR_INVALID_ARG),               # > topk_groups * group size
    (dict(top_k=0), B.MOE_ERR_INVALID_ARG),
    (dict(route_scale=0.0), B.MOE_ERR_INVALID_ARG),
    (dict(route_scale=float("nan")), B.MOE_ERR_INVALID_ARG),
    (dict(route_scale=float("inf")), B.MOE_ERR_INVALID_ARG),
    (dict(dim=0), B.MOE_ERR_INVALID_ARG),
    (dict(n_shared=-1), B.MOE_ERR_INVALID_ARG),
    (dict(score_func=7), B.MOE_ERR_INVALID_ARG),
    (dict(norm_topk=2), B.MOE_ERR_INVALID_ARG),
    (dict(add_residual=3), B.MOE_ERR_INVALID_ARG),
    (dict(act_dtype=B.MOE_F32, weight_dtype=B.MOE_BF16), B.MOE_ERR_UNSUPPORTED),
    (dict(act_dtype=B.MOE_F32, weight_dtype=B.MOE_FP8_E4M3_B128), B.MOE_ERR_UNSUPPORTED),
    (dict(act_dtype=B.MOE_BF16, weight_dtype=B.MOE_FP8_E4M3_B128, inter_dim=192), B.MOE_ERR_UNSUPPORTED),
    (dict(dim=260), B.MOE_ERR_UNSUPPORTED),
    (dict(n_routed=1024, n_groups=1, topk_groups=1), B.MOE_ERR_UNSUPPORTED),
    (dict(n_routed=64, n_groups=1, topk_groups=1, top_k=33), B.MOE_ERR_UNSUPPORTED),
])
def test_invalid_configs_rejected(kw, status):
    with pytest.raises(B.MoeError) as ei:
        B.moe_validate(_cfg(**kw))
    assert ei.value.status == status


def test_entry_points_validate_before_launch():
    """Every failure below is caught on the host; nothing is enqueued."""
    c = _cfg()
    L = B.lib()
    fake = 1 << 20   # aligned, never dereferenced: validation fails first
    # negative T
    assert L.moe_gate(ctypes.byref(c), -1, fake, fake, None, fake, fake, fake, None, None) == B.MOE_ERR_INVALID_ARG
    # NULL inputs / outputs
    assert L.moe_gate(ctypes.byref(c), 4, None, fake, None, fake, fake, fake, None, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_gate(ctypes.byref(c), 4, fake, fake, None, None, fake, fake, None, None) == B.MOE_ERR_INVALID_ARG
    # misaligned pointer
    assert L.moe_gate(ctypes.byref(c), 4, fake + 2, fake, None, fake, fake, fake, None, None) == B.MOE_ERR_INVALID_ARG
    assert b"aligned" in L.moe_last_error()
    # bias with groups of one expert
    c1 = _cfg(n_routed=4, n_groups=4, topk_groups=2, top_k=2)
    assert L.moe_gate(ctypes.byref(c1), 4, fake, fake, fake, fake, fake, fake, None, None) == B.MOE_ERR_INVALID_ARG
    # routing struct built for another T
    r = B.moe_routing_init(c, 64, fake, B.moe_routing_size(c, 64))
    assert L.moe_permute(ctypes.byref(c), 32, fake, ctypes.byref(r), None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_combine(ctypes.byref(c), 32, fake, None, fake, ctypes.byref(r), fake, fake, None) == B.MOE_ERR_INVALID_ARG
    # workspace too small / NULL / misaligned
    w = B.moe_weights(w_gate=fake, w13=fake, w2=fake, sw13=fake, sw2=fake)
    need = B.moe_workspace_size(c, 64)
    assert L.moe_forward(ctypes.byref(c), 64, fake, ctypes.byref(w), fake + 256, None, None, fake, need - 1, None) == B.MOE_ERR_WORKSPACE
    assert L.moe_forward(ctypes.byref(c), 64, fake, ctypes.byref(w), fake + 256, None, None, None, need, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_forward(ctypes.byref(c), 64, fake, ctypes.byref(w), fake + 256, None, None, fake + 16, need, None) == B.MOE_ERR_INVALID_ARG
    # out aliasing x
    assert L.moe_forward(ctypes.byref(c), 64, fake, ctypes.byref(w), fake, None, None, fake, need, None) == B.MOE_ERR_INVALID_ARG
    # missing shared weights when n_shared > 0
    w2 = B.moe_weights(w_gate=fake, w13=fake, w2=fake)
    assert L.moe_forward(ctypes.byref(c), 64, fake, ctypes.byref(w2), fake + 256, None, None, fake, need, None) == B.MOE_ERR_INVALID_ARG
    # fp8 without scales
    c8 = B.config_of(configs.V3_DECODE_FP8)
    need8 = B.moe_workspace_size(c8, 8)
    assert L.moe_forward(ctypes.byref(c8), 8, fake, ctypes.byref(w), fake + 256, None, None, fake, need8, None) == B.MOE_ERR_INVALID_ARG


def test_bias_update_validates_before_launch():
    c = _cfg()
    L = B.lib()
    fake = 1 << 20
    r = B.moe_routing_init(c, 64, fake, B.moe_routing_size(c, 64))
    for gamma in (float("nan"), float("inf"), -1e-3):
        assert L.moe_bias_update(ctypes.byref(c), 64, ctypes.byref(r), gamma, fake, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_bias_update(ctypes.byref(c), 64, ctypes.byref(r), 1e-3, None, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_bias_update(ctypes.byref(c), 64, ctypes.byref(r), 1e-3, fake + 2, None) == B.MOE_ERR_INVALID_ARG
    # routing built for another T
    assert L.moe_bias_update(ctypes.byref(c), 32, ctypes.byref(r), 1e-3, fake, None) == B.MOE_ERR_INVALID_ARG
    r0 = B.moe_routing_init(c, 0, fake, B.moe_routing_size(c, 0))
    assert L.moe_bias_update(ctypes.byref(c), 0, ctypes.byref(r0), 1e-3, fake, None) == B.MOE_OK


def test_balance_loss_validates_before_launch():
    c = _cfg()
    L = B.lib()
    fake = 1 << 20
    one = ctypes.c_float(1.0)
    ws = B.moe_balance_loss_workspace_size(c, 64, 32)
    # per-chunk fp64 partials and int32 counts for 2 sequences x 1 chunk x E experts
    assert ws >= 2 * c.n_routed * 12
    assert B.moe_balance_loss_workspace_size(c, 0, 32) == 0
    call = lambda T, sl, lg, a, w, wb, loss: L.moe_balance_loss(ctypes.byref(c), T, sl, lg, fake, a, w, wb, loss, None)
    assert call(64, 0, fake, one, fake, ws, fake) == B.MOE_ERR_INVALID_ARG       # seq_len < 1
    assert call(64, 48, fake, one, fake, ws, fake) == B.MOE_ERR_INVALID_ARG      # T % seq_len
    assert call(64, 32, fake, ctypes.c_float(float("nan")), fake, ws, fake) == B.MOE_ERR_INVALID_ARG
    assert call(64, 32, None, one, fake, ws, fake) == B.MOE_ERR_INVALID_ARG      # logits NULL
    assert call(64, 32, fake, one, fake, ws, fake + 2) == B.MOE_ERR_INVALID_ARG  # misaligned loss
    assert call(64, 32, fake, one, None, ws, fake) == B.MOE_ERR_INVALID_ARG      # no workspace
    assert call(64, 32, fake, one, fake + 16, ws, fake) == B.MOE_ERR_INVALID_ARG  # misaligned workspace
    assert call(64, 32, fake, one, fake, ws - 1, fake) == B.MOE_ERR_WORKSPACE     # too small
    assert call(0, 32, fake, one, None, 0, fake) == B.MOE_OK                      # T == 0: nothing to do
    with pytest.raises(B.MoeError):
        B.moe_balance_loss_workspace_size(c, 64, 48)


def test_T_zero_is_a_no_op():
    c = _cfg()
    L = B.lib()
    fake = 1 << 20
    assert L.moe_gate(ctypes.byref(c), 0, fake, fake, None, fake, fake, fake, None, None) == B.MOE_OK
    w = B.moe_weights(w_gate=fake, w13=fake, w2=fake, sw13=fake, sw2=fake)
    need = B.moe_workspace_size(c, 0)
    assert L.moe_forward(ctypes.byref(c), 0, fake, ctypes.byref(w), fake + 256, None, None, fake, need, None) == B.MOE_OK
    assert L.moe_last_error() == b""


def test_routing_layout_is_aligned_and_disjoint():
    for shape in configs.ALL:
        c = B.config_of(shape)
        n = B.moe_routing_size(c, shape.T)
        base = 1 << 30
        r = B.moe_routing_init(c, shape.T, base, n)
        P = shape.T * shape.top_k
        spans = sorted([(r.counts, 4 * shape.n_routed), (r.expert_off, 4 * (shape.n_routed + 1)),
                        (r.sorted_pair, 4 * r.max_rows), (r.pair_row, 4 * P),
                        (r.tile_expert, 4 * r.max_tiles), (r.tile_row, 4 * r.max_tiles),
                        (r.n_tiles, 4), (r.scratch, 4)])
        for (a, la), (b, _) in zip(spans, spans[1:]):
            assert a % 256 == 0 and a + la <= b
        assert spans[-1][0] < base + n
        assert r.max_rows % r.tile_m == 0 and r.max_rows >= P + min(P, shape.n_routed) * (r.tile_m - 1)
        assert r.max_tiles * r.tile_m == r.max_rows


def test_backward_validates_before_launch():
    L = B.lib()
    fake = 1 << 20
    c = B.config_of(configs.V2_LITE_BF16)
    T = 64
    need = B.moe_backward_workspace_size(c, T)
    r = B.moe_routing_init(c, T, fake, B.moe_routing_size(c, T))
    w = B.moe_weights(w_gate=fake, w13=fake, w2=fake, sw13=fake, sw2=fake)
    g = B.moe_grads(dx=fake, dw_gate=fake, dw13=fake, dw2=fake, dsw13=fake, dsw2=fake)
    ws = 1 << 32

    def call(cfg=c, T=T, wts=w, grads=g, dout=fake, wsp=ws, nb=need):
        return L.moe_backward(ctypes.byref(cfg), T, fake, ctypes.byref(wts), ctypes.byref(r), fake, fake, fake,
                              fake, dout, ctypes.byref(grads), wsp, nb, None)
    assert call(dout=None) == B.MOE_ERR_INVALID_ARG
    assert call(grads=B.moe_grads(dx=fake, dw_gate=fake, dw13=fake, dw2=None, dsw13=fake, dsw2=fake)) == B.MOE_ERR_INVALID_ARG
    assert call(grads=B.moe_grads(dx=fake, dw_gate=fake, dw13=fake, dw2=fake)) == B.MOE_ERR_INVALID_ARG  # shared grads
    assert call(wsp=None) == B.MOE_ERR_INVALID_ARG
    assert call(wsp=ws + 64) == B.MOE_ERR_INVALID_ARG
    assert call(nb=need - 1) == B.MOE_ERR_WORKSPACE
    assert call(dout=fake + 8) == B.MOE_ERR_INVALID_ARG                    # 16-byte alignment
    assert L.moe_backward(ctypes.byref(c), T, fake, ctypes.byref(w), ctypes.byref(r), fake + 2, fake, fake,
                          fake, fake, ctypes.byref(g), ws, need, None) == B.MOE_ERR_INVALID_ARG   # misaligned topk_idx
    for bad in (B.config_of(configs.TINY_F32), B.config_of(configs.V3_DECODE_FP8)):
        with pytest.raises(B.MoeError) as ei:
            B.moe_backward_workspace_size(bad, 8)
        assert ei.value.status == B.MOE_ERR_UNSUPPORTED
    r0 = B.moe_routing_init(c, 0, fake, B.moe_routing_size(c, 0))
    assert L.moe_backward(ctypes.byref(c), 0, fake, ctypes.byref(w), ctypes.byref(r0), fake, fake, fake, fake,
                          fake, ctypes.byref(g), None, 0, None) == B.MOE_OK
    # the workspace grows with T and holds the 128-row tile lists, fp32 a/c, dh, dx per routed row
    assert B.moe_backward_workspace_size(c, 2 * T) > need


def test_saved_preactivation_entry_points_validate_before_launch():
    L = B.lib()
    fake = 1 << 20
    c = B.config_of(configs.V2_LITE_BF16)   # two shared experts
    T = 64
    need = B.moe_backward_workspace_size(c, T)
    r = B.moe_routing_init(c, T, fake, B.moe_routing_size(c, T))
    w = B.moe_weights(w_gate=fake, w13=fake, w2=fake, sw13=fake, sw2=fake)
    g = B.moe_grads(dx=fake, dw_gate=fake, dw13=fake, dw2=fake, dsw13=fake, dsw2=fake)
    ws = 1 << 32

    def ffn(cfg=c, T=T, ab=fake, abs_=fake, hs=fake):
        return L.moe_expert_ffn_save(ctypes.byref(cfg), T, fake, ctypes.byref(r), ctypes.byref(w), fake, fake,
                                     hs, fake, ab, abs_, None)

    def bwd(ab=fake, abs_=fake, nb=need):
        return L.moe_backward_saved(ctypes.byref(c), T, fake, ctypes.byref(w), ctypes.byref(r), fake, fake,
                                    fake, fake, fake, ab, abs_, ctypes.byref(g), ws, nb, None)
    assert ffn(ab=None) == B.MOE_ERR_INVALID_ARG
    assert ffn(ab=fake + 4) == B.MOE_ERR_INVALID_ARG                # 16-byte alignment
    assert ffn(abs_=None) == B.MOE_ERR_INVALID_ARG                  # a shared expert needs abs
    assert ffn(hs=None) == B.MOE_ERR_INVALID_ARG
    assert ffn(cfg=B.config_of(configs.V3_DECODE_FP8), T=8) == B.MOE_ERR_UNSUPPORTED   # bf16 only
    assert bwd(ab=None) == B.MOE_ERR_INVALID_ARG
    assert bwd(abs_=None) == B.MOE_ERR_INVALID_ARG
    assert bwd(abs_=fake + 8) == B.MOE_ERR_INVALID_ARG
    assert bwd(nb=need - 1) == B.MOE_ERR_WORKSPACE
    r0 = B.moe_routing_init(c, 0, fake, B.moe_routing_size(c, 0))
    assert L.moe_expert_ffn_save(ctypes.byref(c), 0, fake, ctypes.byref(r0), ctypes.byref(w), fake, fake,
                                 fake, fake, fake, fake, None) == B.MOE_OK


def test_static_forward_rejects_layers_beyond_its_scratch():
    """moe_forward_static checks its workspace need against the static array on the
    host, before any device call: the V3 prefill batch needs far more than 64 MiB."""
    import torch
    shape = configs.V3_PREFILL_BF16
    cfg = B.config_of(shape)
    assert B.moe_workspace_size(cfg, shape.T) > 64 << 20
    x = torch.zeros(16)
    with pytest.raises(B.MoeError) as ei:
        B.moe_forward_static(cfg, shape.T, x, B.moe_weights(), x, stream=0)
    assert ei.value.status == B.MOE_ERR_WORKSPACE
    assert "static" in B.lib().moe_last_error().decode()
    bad = B.config_of(shape.with_(n_groups=3))
    with pytest.raises(B.MoeError) as ei:
        B.moe_forward_static(bad, 8, x, B.moe_weights(), x, stream=0)
    assert ei.value.status == B.MOE_ERR_INVALID_ARG
