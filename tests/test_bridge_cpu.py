"""The test glue's two weight converters give the same exact float64 values.

tests/oracle_bridge.py decodes stored weights through the oracle's own
decoders; for full-size layers it can instead let torch convert them (bf16 and
fp32 widen exactly, and an e4m3 code times its fp32 block scale is exact in
float64).  Both must agree bit for bit on every storage format."""
import numpy as np
import pytest

from oracle_bridge import weight_f64, weight_f64_torch
from routed_expert_moe_amd import configs, synth


@pytest.mark.parametrize("kind", ["f32", "bf16", "fp8"])
def test_fast_weight_conversion_is_exact(kind):
    base = configs.V3_DECODE_FP8 if kind == "fp8" else configs.TINY_F32
    s = base.with_(name=f"bridge_{kind}", T=4, n_routed=2, n_groups=1, topk_groups=1, top_k=1,
                   dim=256, inter_dim=256, weight=kind, act="f32" if kind == "f32" else "bf16")
    layer = synth.make_layer(s, device="cpu")
    for e in range(2):
        for q, sc in ((layer.w13[e], None if kind != "fp8" else layer.w13_scale[e]),
                      (layer.w2[e], None if kind != "fp8" else layer.w2_scale[e])):
            a, b = weight_f64(q, sc, kind), weight_f64_torch(q, sc, kind)
            assert a.dtype == b.dtype == np.float64
            assert np.array_equal(a.view(np.uint64), b.view(np.uint64))
