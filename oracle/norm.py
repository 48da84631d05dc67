"""BF16 RMSNorm followed by per-token FP8 quantization — test infrastructure
only.

Sources.  MOSS-VL-Realtime-FP8 article, component / precision map: the
language model's norms are RMSNorm and stay in BF16, while the q/k/v and
gate/up projections they feed are FP8_DYNAMIC Linears, whose first step is
the per-token quantization of exactly the norm's output row (README,
"FP8-Dynamic").  MOSS-VL-Instruct-0708-FP8 tuning checklist: norms are among
the modules kept in BF16.

Readings where the pages are silent (plainest reading the rest supports):

* RMSNorm of a row x with weight gamma: ``x / sqrt(mean(x^2) + eps)``
  scaled elementwise by gamma; ``eps`` is a caller's parameter;
* "stays BF16" is read as two bfloat16 roundings, as a BF16 norm module
  produces them: the normalized row ``t = bf16(x / sqrt(mean(x^2) + eps))``,
  then ``y = bf16(gamma * t)`` (gamma is bfloat16, so the product of two
  8-bit significands is exact before that rounding);
* the normalization itself is evaluated in float64 here (the kernel's
  float32 evaluation may land on the other side of a bfloat16 rounding
  boundary for a few elements: the tests compare ``y`` within one bfloat16
  step and the quantized bytes exactly, given the same ``y``);
* the quantization of ``y`` is :func:`oracle.quant.quant_act_ref`.
"""

import numpy as np

from .bf16 import bf16_bits_to_f32, f64_to_bf16_bits
from .quant import quant_act_ref


def rmsnorm_ref(x_bf16_bits: np.ndarray, gamma_bf16_bits: np.ndarray, eps: float):
    """RMSNorm of each row of X[M, K] (bf16 bits) with weight gamma[K].

    Returns ``(y_bits uint16 [M, K], t_f64 [M, K])``: the bfloat16 output and
    the unrounded normalized rows ``x / sqrt(mean(x^2) + eps)`` in float64.
    Step 1: ``ms[m] = sum_k x[m,k]^2 / K`` (each square exact in float64).
    Step 2: ``t = x / sqrt(ms + eps)``, rounded to bfloat16.
    Step 3: ``y = bf16(gamma * bf16(t))`` (the product is exact in float64).
    """
    x = bf16_bits_to_f32(np.asarray(x_bf16_bits, np.uint16)).astype(np.float64)
    g = bf16_bits_to_f32(np.asarray(gamma_bf16_bits, np.uint16)).astype(np.float64)
    if x.ndim != 2 or g.ndim != 1 or g.shape[0] != x.shape[1]:
        raise ValueError("expected X[M, K] and gamma[K]")
    if not (np.all(np.isfinite(x)) and np.all(np.isfinite(g))):
        raise ValueError("inputs must be finite")
    if not (eps >= 0.0 and np.isfinite(eps)):
        raise ValueError("eps must be finite and non-negative")
    if x.shape[1] == 0:
        return np.zeros(x.shape, np.uint16), np.zeros(x.shape)
    ms = np.sum(x * x, axis=1) / x.shape[1]                      # step 1
    denom = np.sqrt(ms + eps)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(denom[:, None] > 0, x / denom[:, None], 0.0 * x)   # step 2
    t_bits = f64_to_bf16_bits(t)
    y = g[None, :] * bf16_bits_to_f32(t_bits).astype(np.float64)     # step 3
    return f64_to_bf16_bits(y), t


def rmsnorm_quant_ref(x_bf16_bits: np.ndarray, gamma_bf16_bits: np.ndarray,
                      eps: float):
    """RMSNorm then per-token quantization of its bfloat16 output.

    Returns ``(qx uint8 [M, K], s_x f32 [M], y_bits uint16 [M, K])``.
    """
    y_bits, _ = rmsnorm_ref(x_bf16_bits, gamma_bf16_bits, eps)
    qx, sx = quant_act_ref(y_bits)
    return qx, sx, y_bits
