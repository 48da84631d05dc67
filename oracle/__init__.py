"""CPU oracle for the FP8_DYNAMIC W8A8 Linear — TEST INFRASTRUCTURE ONLY.

This package is the slow, plainly written reference that the HIP path is
checked against.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; the product path
(``fp8_w8a8_dynamic_amd``) never does, and it shares no code with it.

What it computes follows the MOSS-VL quantization README (the
"FP8-Dynamic" recipe section: ``float8_e4m3fn`` weights with channel-wise
static scales, activations quantized to FP8 per token at run time) and the
MOSS-VL-Realtime-FP8 article (the section explaining why the 252 Linears use
FP8 E4M3: 4 exponent bits, 3 mantissa bits, offline per-channel weight
scales, dynamic per-token activation scales).  The pages give no formula for
the scale, the rounding mode or the accumulator; the readings used here
(scale = amax/448 in fp32, IEEE fp32 division, round-to-nearest-even with
saturation, fp64 accumulation, token-scale x channel-scale epilogue) are
listed where each function is defined.

Modules
-------
e4m3    256-entry decode table and the nearest-value encoder.
quant   per-token activation and per-output-channel weight quantization.
linear  fp64 matmul of decoded codes and the scale epilogue.
norm    BF16 RMSNorm and the per-token quantization of its output (the
        fusion ahead of the q/k/v and gate/up Linears).
swiglu  the SiLU-gated activation between gate/up and down and the
        per-token quantization of its output (down_proj's input).
kvcache the FP8 E4M3 key/value-cache codec (group-wise dynamic scales,
        float32 read-back rounded to bf16) and the INT8 group-wise cache
        with a BF16 residual window (asymmetric min-max reading of HQQ).
tiles   the MFMA-tile order of weight codes read by the grouped few-token
        call (a byte permutation of the library's own).
check   the pass criteria (bit-exact bytes, elementwise output tolerance).

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
(closed forms, hand-derived golden values, brute force in exact rational
arithmetic, torch's independent CPU ``float8_e4m3fn`` cast, and torch's
float64 ``rms_norm`` for the normalization, scipy's ``expit`` and
50-digit decimal arithmetic for the activation).
"""

from .e4m3 import (DECODE_TABLE, FINITE_MAX, decode, encode, encode_exact,
                   POSITIVE_VALUES)
from .bf16 import bf16_bits_to_f32, f64_to_bf16_bits
from .quant import quant_act_ref, quant_weight_ref, quant_rows_ref
from .linear import linear_ref, quant_linear_ref
from .tiles import tile_weights_ref
from .check import check_bytes, check_close, close_report

__all__ = [
    "DECODE_TABLE", "FINITE_MAX", "POSITIVE_VALUES", "decode", "encode",
    "encode_exact", "bf16_bits_to_f32", "f64_to_bf16_bits", "quant_act_ref",
    "quant_weight_ref", "quant_rows_ref", "linear_ref", "quant_linear_ref",
    "tile_weights_ref", "check_bytes", "check_close", "close_report",
]
