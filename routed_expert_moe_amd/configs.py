"""Named DeepSeekMoE layer shapes and their synthetic-input recipes.

A `LayerShape` carries the arguments that define one MoE layer forward
(dim, n_routed, n_shared, n_groups, topk_groups, top_k, route_scale,
inter_dim, score function) plus the storage precision and the recipe the
seeded input generator uses for it.  It holds no arithmetic of the method.

The MoE fields of the V3-shaped layers come from the model.py config table on
the DeepSeek-V3 notes page (73biji.xyz/llm_pp_dsv3, "DeepSeek-V3 (model.py
config)" table: dim 7168, 256 routed + 1 shared experts, 8 activated, 8 groups
with 4 kept, route_scale 2.5, sigmoid scoring, fp8 weights).  The V2-shaped
layer takes hidden size 5120, 160 routed experts, top-6 and 2 shared experts
from the DeepSeek-V2 model card (aigallery-kappa.vercel.app/models/deepseek-v2,
architecture sketch).  The pages give no expert hidden size (inter_dim) and no
V2-Lite shape; those values are part of the workload definition this library
is measured on.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import Optional

SCORE_SIGMOID = "sigmoid"
SCORE_SOFTMAX = "softmax"


@dataclass(frozen=True)
class LayerShape:
    name: str
    T: int                     # tokens in one call
    dim: int                   # model hidden size
    n_routed: int              # routed experts E
    n_groups: int              # routing groups G (1 = no group limit)
    topk_groups: int           # groups kept per token
    top_k: int                 # experts activated per token K
    n_shared: int              # shared experts S (fused into one FFN of S*inter_dim)
    inter_dim: int             # hidden size I of one expert FFN
    score: str                 # "sigmoid" | "softmax"
    route_scale: float
    act: str                   # activation / gate-weight storage: "f32" | "bf16"
    weight: str                # expert weight storage: "f32" | "bf16" | "fp8"
    norm_topk: int = -1        # -1: sigmoid renormalises, softmax does not
    add_residual: int = 1
    act_quant: int = 0         # 1: FP8 W8A8 (activations quantised 1x128 before the expert GEMMs)
    # --- synthetic input recipe ---
    seed: int = 0
    bias_range: Optional[float] = None   # per-expert bias ~ U(-r, r); None = no bias
    zipf: Optional[float] = None         # gate rows scaled by a seeded Zipf(s) profile

    @property
    def pairs(self) -> int:
        return self.T * self.top_k

    def with_(self, **kw) -> "LayerShape":
        return dataclasses.replace(self, **kw)


TINY_F32 = LayerShape(
    name="tiny_f32", T=64, dim=256, n_routed=16, n_groups=4, topk_groups=2,
    top_k=4, n_shared=1, inter_dim=128, score=SCORE_SIGMOID, route_scale=2.5,
    act="f32", weight="f32", seed=0, bias_range=0.1)

V2_LITE_BF16 = LayerShape(
    name="v2lite_bf16_T512", T=512, dim=2048, n_routed=64, n_groups=1,
    topk_groups=1, top_k=6, n_shared=2, inter_dim=1408, score=SCORE_SOFTMAX,
    route_scale=1.0, act="bf16", weight="bf16", seed=1, zipf=1.1)

V2_BF16 = LayerShape(
    name="v2_bf16_T4096", T=4096, dim=5120, n_routed=160, n_groups=1,
    topk_groups=1, top_k=6, n_shared=2, inter_dim=1536, score=SCORE_SOFTMAX,
    route_scale=1.0, act="bf16", weight="bf16", seed=2)

V3_PREFILL_BF16 = LayerShape(
    name="v3_prefill_bf16_T8192", T=8192, dim=7168, n_routed=256, n_groups=8,
    topk_groups=4, top_k=8, n_shared=1, inter_dim=2048, score=SCORE_SIGMOID,
    route_scale=2.5, act="bf16", weight="bf16", seed=3, bias_range=0.05)

V3_DECODE_FP8 = LayerShape(
    name="v3_decode_fp8_T8", T=8, dim=7168, n_routed=256, n_groups=8,
    topk_groups=4, top_k=8, n_shared=1, inter_dim=2048, score=SCORE_SIGMOID,
    route_scale=2.5, act="bf16", weight="fp8", seed=4, bias_range=0.05)

# The V3 prefill batch with the released checkpoint's fp8 expert weights and the
# W8A8 expert format (a next step after the bf16 and decode workloads).
V3_PREFILL_W8A8 = LayerShape(
    name="v3_prefill_w8a8_T8192", T=8192, dim=7168, n_routed=256, n_groups=8,
    topk_groups=4, top_k=8, n_shared=1, inter_dim=2048, score=SCORE_SIGMOID,
    route_scale=2.5, act="bf16", weight="fp8", act_quant=1, seed=5, bias_range=0.05)

# One GPU's share of the V3 prefill layer under expert parallelism over the 8
# GPUs of a node (one routing group of 32 experts per GPU): the 8192 tokens'
# 65536 pairs split eight ways, each token reaching at most 4 GPUs, so a GPU
# receives about 4096 distinct tokens with 2 of its experts each, 256 rows per
# expert as in the whole layer.  The shared expert runs on the tokens' home GPU.
V3_EP_SHARD_BF16 = LayerShape(
    name="v3_ep_shard_bf16_T4096_E32", T=4096, dim=7168, n_routed=32, n_groups=1,
    topk_groups=1, top_k=2, n_shared=0, inter_dim=2048, score=SCORE_SIGMOID,
    route_scale=2.5, act="bf16", weight="bf16", seed=6, bias_range=0.05)

ALL = [TINY_F32, V2_LITE_BF16, V2_BF16, V3_PREFILL_BF16, V3_DECODE_FP8, V3_PREFILL_W8A8, V3_EP_SHARD_BF16]
BY_NAME = {c.name: c for c in ALL}
