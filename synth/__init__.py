"""Seeded synthetic workloads shared by the tests and the benchmark."""
from .configs import CONFIGS, ORDER, LayerConfig, scaled
from .inputs import (LayerInputs, make_fp8_experts, make_inputs, make_logits, make_bias,
                     to_bf16_bits)

__all__ = ["CONFIGS", "ORDER", "LayerConfig", "scaled", "LayerInputs",
           "make_inputs", "make_fp8_experts", "make_logits", "make_bias", "to_bf16_bits"]
