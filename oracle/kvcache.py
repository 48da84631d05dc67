"""FP8 E4M3 key/value-cache codec — test infrastructure only.

Source.  MOSS-VL quantization README, "KV cache": the KV cache keeps growing
with a video stream, so it is quantized at generation time; with the FP8
checkpoint under SGLang the engine's own KV dtype is used, e.g.
``--kv-cache-dtype fp8_e4m3``.  The pages give only that dtype.

Readings where the pages are silent (plainest reading the rest supports):

* the cache stores each token's K (and V) row, ``kv_heads * head_dim``
  values, as E4M3 codes with the same encoder as the activations
  (:mod:`oracle.quant`: amax, ``scale = fl32(amax / 448)``, IEEE float32
  quotient, round to nearest even, saturation, signed zeros);
* one float32 scale per (token, group of ``group`` consecutive values),
  computed when the token is written (dynamic, as the FP8-Dynamic recipe does
  for activations; a static scale would have to be calibrated, and the
  recipe uses no calibration data); the default group is one KV head
  (head_dim = 128 values);
* reading the cache gives ``bf16(fl32(dec(code) * scale))``: the product in
  float32, then one rounding to bfloat16, the dtype attention computes in.
"""

import numpy as np

from .bf16 import f64_to_bf16_bits
from .e4m3 import DECODE_TABLE
from .quant import quant_act_ref


def _check_group(width: int, group: int):
    if group < 1 or width % group != 0:
        raise ValueError("the row width must be a multiple of the group")


def kv_fp8_quant_ref(kv_bf16_bits: np.ndarray, group: int):
    """Quantize rows of K or V [R, W] (bf16 bits) in groups of ``group``.

    Returns ``(codes uint8 [R, W], scales float32 [R, W // group])``; each
    group is quantized exactly as one row of :func:`quant_act_ref`.
    """
    x = np.asarray(kv_bf16_bits, np.uint16)
    if x.ndim != 2:
        raise ValueError("expected K or V rows [R, W]")
    r, w = x.shape
    _check_group(w, group)
    codes, scales = quant_act_ref(x.reshape(r * (w // group), group))
    return codes.reshape(r, w), scales.reshape(r, w // group)


def kv_fp8_dequant_ref(codes: np.ndarray, scales: np.ndarray, group: int):
    """bf16 bits [R, W] of ``bf16(fl32(dec(code) * scale))``.

    ``dec`` is the oracle's decode table (exact in float32: at most 4
    significant bits); the product is one IEEE float32 multiplication (numpy
    float32), then one rounding to nearest-even bfloat16.
    """
    c = np.asarray(codes, np.uint8)
    s = np.asarray(scales, np.float32)
    r, w = c.shape
    _check_group(w, group)
    if s.shape != (r, w // group):
        raise ValueError("one scale per group")
    dec = DECODE_TABLE.astype(np.float32)[c]
    prod = dec * np.repeat(s, group, axis=1)
    assert prod.dtype == np.float32
    return f64_to_bf16_bits(prod.astype(np.float64))
