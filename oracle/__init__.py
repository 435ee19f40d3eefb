"""CPU float64 oracle for the DeepSeekMoE layer (forward, backward, balance terms, W8A8).

TEST INFRASTRUCTURE: imported only by the tests, the package entry file's smoke
check and the benchmark's CPU-baseline leg.  The library never imports it.
"""
from .moe_oracle import (Spec, GateResult, decode_bf16, decode_e4m3, dequant_e4m3_block128,
                         gate, gate_logits, gate_scores, group_scores, moe_layer,
                         route_weights, select_experts, selection_margins, sigmoid, silu,
                         swiglu_ffn, swiglu_preacts)

__all__ = ["Spec", "GateResult", "decode_bf16", "decode_e4m3", "dequant_e4m3_block128", "gate",
           "gate_logits", "gate_scores", "group_scores", "moe_layer", "route_weights",
           "select_experts", "selection_margins", "sigmoid", "silu", "swiglu_ffn", "swiglu_preacts"]
