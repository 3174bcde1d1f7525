"""Seeded synthetic inputs for the FLARE++ mixer (shared by the oracle tests, the GPU tests and the bench).

This package draws random tensors and casts them to their storage dtype. It holds none of the
mixer's arithmetic: no normalization, no softmax, no contraction.
"""
from .gen import (CONFIGS, DESCRIPTIONS, FAMILIES, BlockInputs, Workload, make_block_inputs, make_workload, make_cotangent, make_synthesis_values,
                  bf16_bits_from_float,
                  float_from_bf16_bits, to_float64, workload_seed)

__all__ = ["CONFIGS", "DESCRIPTIONS", "FAMILIES", "BlockInputs", "Workload", "make_block_inputs", "make_workload", "make_cotangent", "make_synthesis_values", "bf16_bits_from_float", "float_from_bf16_bits",
           "to_float64", "workload_seed"]
