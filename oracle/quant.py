"""Per-token and per-output-channel FP8 quantization of the CPU oracle.

Test infrastructure only.

Sources.  MOSS-VL quantization README, "FP8-Dynamic" recipe: weights are
``float8_e4m3fn`` with channel-wise static scales, and the activations that
enter the quantized kernels are quantized to FP8 per token, dynamically.
MOSS-VL-Realtime-FP8 article, section on why the 252 Linears use FP8 E4M3:
weight scales are computed offline per channel ("zero runtime overhead"),
activation scales are computed per token at run time because activations
drift and carry outliers.  The README also says the recipe uses no
calibration data, so the weight scale can only come from the weight itself.

Readings where the pages are silent (each one is the plainest reading that
the rest supports):

* symmetric scaling, no zero point: ``scale = amax / 448`` where ``amax`` is
  the largest magnitude of the row and 448 the largest finite E4M3 value;
* the scale is a float32, computed by one IEEE float32 division;
* each element is divided by the scale with one IEEE float32 division and
  the float32 quotient is encoded to E4M3 by round-to-nearest-even with
  saturation at +-448 (:func:`oracle.e4m3.encode`);
* "channel" means output channel, i.e. a row of ``W[out, in]``: only
  per-output-channel and per-token scales factor out of the sum over the
  input dimension, which the token-scale x channel-scale epilogue needs;
* a row whose amax is 0 gets scale 0 and codes +-0 (sign kept), with no
  0/0 division;
* no flush of subnormals anywhere (a tiny row keeps its subnormal scale).
"""

import numpy as np

from .bf16 import bf16_bits_to_f32
from .e4m3 import FINITE_MAX, encode


def quant_rows_ref(rows_f32: np.ndarray):
    """Quantize each row of a float32 matrix with its own scale.

    Returns ``(codes uint8 [R, C], scales float32 [R])``.
    Step 1: ``amax[r] = max_c |x[r, c]|`` (exact in float32).
    Step 2: ``scale[r] = fl32(amax[r] / 448)``.
    Step 3: ``code[r, c] = enc(fl32(x[r, c] / scale[r]))``.
    """
    x = np.asarray(rows_f32, dtype=np.float32)
    if x.ndim != 2:
        raise ValueError("expected a 2-D matrix of rows")
    if not np.all(np.isfinite(x)):
        raise ValueError("inputs must be finite")
    rows, cols = x.shape
    if cols == 0:
        return np.zeros((rows, 0), np.uint8), np.zeros(rows, np.float32)
    amax = np.max(np.abs(x), axis=1)                          # step 1
    scale = amax / np.float32(FINITE_MAX)                      # step 2
    assert scale.dtype == np.float32
    zero_row = scale == 0
    safe = np.where(zero_row, np.float32(1.0), scale).astype(np.float32)
    quotient = x / safe[:, None]                               # step 3
    assert quotient.dtype == np.float32
    # amax == 0: every element is +-0, keep it as is (sign-preserving zero).
    quotient = np.where(zero_row[:, None], x, quotient)
    codes = encode(quotient)
    return codes, scale.astype(np.float32)


def quant_act_ref(x_bf16_bits: np.ndarray):
    """Per-token dynamic quantization of activations ``X[M, K]`` (bf16 bits).

    One scale per token (row).  Returns ``(qx uint8 [M, K], s_x f32 [M])``.
    """
    x = bf16_bits_to_f32(np.asarray(x_bf16_bits, dtype=np.uint16))
    return quant_rows_ref(x)


def quant_weight_ref(w_bf16_bits: np.ndarray):
    """Channel-wise static quantization of weights ``W[N, K]`` (bf16 bits).

    One scale per output channel (row of ``W[out, in]``), computed once,
    offline.  Returns ``(qw uint8 [N, K], s_w f32 [N])``.
    """
    w = bf16_bits_to_f32(np.asarray(w_bf16_bits, dtype=np.uint16))
    return quant_rows_ref(w)
