"""CPU oracle (test infrastructure only; see moe_oracle's module docstring)."""
from .moe_oracle import (bf16_to_f32, f32_to_bf16_rne, quantile, router_logits,
                         route, mixture_weights, eqb_keys_values, eqb_expert_bias,
                         group_by_expert, silu, swiglu, moe_combine, max_vio,
                         intervention_rate, moe_layer)

__all__ = ["bf16_to_f32", "f32_to_bf16_rne", "quantile", "router_logits", "route",
           "mixture_weights", "eqb_keys_values", "eqb_expert_bias",
           "group_by_expert", "silu", "swiglu", "moe_combine", "max_vio",
           "intervention_rate", "moe_layer"]
