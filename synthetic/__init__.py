"""Seeded synthetic inputs shared by the oracle's tests, the GPU tests and the bench."""
from .delta import DeltaInputs, make_delta_dout, make_delta_inputs, make_kda_inputs
from .microbatch import (CONFIGS, Config, Microbatch, bf16_bits_to_f32, f32_to_bf16_bits,
                         make_custom, make_layer, make_microbatch, make_cu_seqlens)

__all__ = ["CONFIGS", "Config", "DeltaInputs", "Microbatch", "make_delta_dout", "make_delta_inputs", "make_kda_inputs", "bf16_bits_to_f32", "f32_to_bf16_bits",
           "make_custom", "make_layer", "make_microbatch", "make_cu_seqlens"]
