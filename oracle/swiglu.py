"""SiLU-gated MLP activation followed by per-token FP8 quantization of the
down projection's input — test infrastructure only.

Sources.  MOSS-VL quantization README, "FP8-Dynamic": gate_proj, up_proj and
down_proj are FP8_DYNAMIC Linears, so the input of down_proj is quantized
per token at run time; the quantization config's packed-module mapping packs
gate_proj and up_proj into one gate_up_proj.  MOSS-VL-Realtime-FP8 article,
component / precision map: everything that is not one of those Linears stays
BF16, which includes the activation between them.

Readings where the pages are silent (plainest reading the rest supports):

* the activation is the SiLU-gated unit of the language model's MLP,
  ``h = silu(gate) * up`` with ``silu(g) = g / (1 + exp(-g))``; the pages
  name gate/up/down projections but not the function, so this is a reading;
* "stays BF16" is read as a BF16 module's two roundings:
  ``s = bf16(silu(g))``, then ``h = bf16(s * u)`` (both factors bfloat16, so
  the product is exact before that rounding);
* silu is evaluated in float64 here;
* the quantization of ``h`` is :func:`oracle.quant.quant_act_ref`.
"""

import numpy as np

from .bf16 import bf16_bits_to_f32, f64_to_bf16_bits
from .quant import quant_act_ref


def silu_f64(g: np.ndarray) -> np.ndarray:
    """``g / (1 + exp(-g))`` in float64 (exp(-g) may overflow to inf for very
    negative g, giving the correct signed-zero limit)."""
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def swiglu_ref(gate_bf16_bits: np.ndarray, up_bf16_bits: np.ndarray):
    """``h = bf16(bf16(silu(gate)) * up)`` elementwise over [M, I] bf16 bits.

    Returns ``(h_bits uint16, s_bits uint16, silu_f64)``: the output, the
    rounded activation and the unrounded activation.
    """
    g = bf16_bits_to_f32(np.asarray(gate_bf16_bits, np.uint16)).astype(np.float64)
    u = bf16_bits_to_f32(np.asarray(up_bf16_bits, np.uint16)).astype(np.float64)
    if g.shape != u.shape:
        raise ValueError("gate and up must have one shape")
    if not (np.all(np.isfinite(g)) and np.all(np.isfinite(u))):
        raise ValueError("inputs must be finite")
    a = silu_f64(g)
    s_bits = f64_to_bf16_bits(a)
    h = bf16_bits_to_f32(s_bits).astype(np.float64) * u
    return f64_to_bf16_bits(h), s_bits, a


def swiglu_quant_ref(gate_bf16_bits: np.ndarray, up_bf16_bits: np.ndarray):
    """The activation, then per-token quantization of its bfloat16 output.

    Returns ``(qh uint8 [M, I], s_h f32 [M], h_bits uint16 [M, I])``.
    """
    h_bits, _, _ = swiglu_ref(gate_bf16_bits, up_bf16_bits)
    qh, sh = quant_act_ref(h_bits)
    return qh, sh, h_bits
