"""fp64 CPU oracle of the DeepSeekMoE layer forward.

Test infrastructure only: the tests, the smoke check and the benchmark's CPU
baseline leg may use it; the product path never does.
"""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import (bf16_bits_to_f64, e4m3_bits_to_f64, dequant_fp8_blocks, widen,
                         router_logits, router_scores, group_limit, topk_select,
                         gate_values, route, exclude_experts, bias_update,
                         stable_permutation, swiglu,
                         expert_weights64, combine_outputs, forward)
