"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle runs.

This package only draws random numbers and rounds them to bfloat16 input
tensors; it contains none of the quantization or matmul arithmetic.  Both the
HIP path and the CPU oracle consume the same host bytes produced here.
"""

from .generators import (LAYER_SHAPES, LINEAR_NAMES, bf16_from_f64, c1_inputs,
                         c2_inputs, c3_inputs, c4_x0, c5_inputs, kv_inputs, norm_inputs,
                         normal_bf16, swiglu_inputs, weight_bf16, rng_for)

__all__ = ["LAYER_SHAPES", "LINEAR_NAMES", "bf16_from_f64", "c1_inputs",
           "c2_inputs", "c3_inputs", "c4_x0", "c5_inputs", "kv_inputs", "norm_inputs",
           "normal_bf16", "swiglu_inputs", "weight_bf16", "rng_for"]
