"""FP8 x FP8 matmul and scale epilogue of the CPU oracle — test infrastructure.

Sources.  MOSS-VL quantization README, "FP8-Dynamic" recipe: the FP8
activations feed "the quantized kernels" together with the FP8 channel-wise
weights; everything outside those Linears stays bfloat16 and the recipe runs
at ``precision="bfloat16"``.  The pages state neither the accumulator nor the
epilogue.  Readings: the product of the decoded codes is summed over the
input dimension; the sum is multiplied by the token's scale and by the
output channel's scale; there is no bias (none is mentioned anywhere); the
layer's output is bfloat16.

The oracle sums in float64.  Every decoded code is a dyadic number with at
most 4 significant bits, so each product is exact in float64 and the only
error is float64 summation, bounded by ``K * 2^-53 * sum|terms|``.
Layouts follow the PyTorch Linear convention: ``X[M, K]``, ``W[N, K]``
(``[out, in]``), ``Y[M, N]``, all row-major.
"""

import numpy as np

from .e4m3 import DECODE_TABLE
from .quant import quant_act_ref


def linear_ref(qx: np.ndarray, s_x: np.ndarray, qw: np.ndarray,
               s_w: np.ndarray) -> np.ndarray:
    """``Y64[m, n] = (sum_k dec(qx[m, k]) * dec(qw[n, k])) * s_x[m] * s_w[n]``.

    Returns the float64 result (the value the GPU's bfloat16 output is
    compared with).
    """
    qx = np.asarray(qx, dtype=np.uint8)
    qw = np.asarray(qw, dtype=np.uint8)
    if qx.ndim != 2 or qw.ndim != 2 or qx.shape[1] != qw.shape[1]:
        raise ValueError("need qx [M, K] and qw [N, K] with the same K")
    s_x = np.asarray(s_x, dtype=np.float32).astype(np.float64)
    s_w = np.asarray(s_w, dtype=np.float32).astype(np.float64)
    if s_x.shape != (qx.shape[0],) or s_w.shape != (qw.shape[0],):
        raise ValueError("one scale per row of qx and per row of qw")
    a = DECODE_TABLE[qx]             # [M, K] float64
    b = DECODE_TABLE[qw]             # [N, K] float64
    if np.isnan(a).any() or np.isnan(b).any():
        raise ValueError("NaN code in an operand")
    acc = a @ b.T                    # [M, N], fp64 sum over k
    return acc * s_x[:, None] * s_w[None, :]


def quant_linear_ref(x_bf16_bits: np.ndarray, qw: np.ndarray,
                     s_w: np.ndarray):
    """Whole FP8_DYNAMIC forward: quantize X per token, then :func:`linear_ref`.

    Returns ``(y64, qx, s_x)``.
    """
    qx, s_x = quant_act_ref(x_bf16_bits)
    return linear_ref(qx, s_x, qw, s_w), qx, s_x
