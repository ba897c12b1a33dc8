"""CPU oracle for the MoE layer forward (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this package. The GPU path never does.
"""
from .moe_oracle import (  # noqa: F401
    Grouping, LayerResult, Routing, balance_stat, bf16_round, capacity_keep, expert_counts,
    forward_grouped, forward_per_token, group, moe_layer, route, router_logits, silu, softmax,
    swiglu_expert, topk_order,
)
