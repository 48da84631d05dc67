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


# ---------------------------------------------------------------------------
# INT8 group-wise KV cache with a BF16 residual window.
#
# Sources.  MOSS-VL quantization README, "KV cache": for Transformers the
# packaging script writes an HQQ INT8 KV-cache config (8 bits, group size
# 64, residual length 128) into generation_config.json, and with
# Transformers' quantized cache the older entries are stored quantized while
# only a short BF16 tail stays unquantized, so reading the cache dequantizes
# the history and concatenates it with that tail.  MOSS-VL-Realtime-FP8
# article, section on the KV cache: K/V compressed to 8-bit integers, every
# 64 elements sharing one set of scaling coefficients, and the most recent
# 128 positions kept in BF16.
#
# Readings (the pages give no formulas; HQQ's solver is not on them):
# * asymmetric min-max per group of `group` consecutive values of a token's
#   row (the starting point of HQQ's fit, without its iterative refinement):
#   mn = min, mx = max (a zero extreme taken as +0: affine codes keep no sign
#   of zero), scale = fl32(fl32(mx - mn) / 255), codes uint8
#   q = clamp(rne(fl32(fl32(x - mn) / scale)), 0, 255); a constant group
#   (scale 0) gets q = 0;
# * reading back: bf16(fl32(fl32(q * scale) + mn)), each step one IEEE
#   float32 operation (no fused multiply-add);
# * the cache holds tokens older than the newest `residual` (128) in this
#   form and the newest ones as plain bf16; reading it yields the
#   dequantized history followed by the bf16 tail.
# ---------------------------------------------------------------------------

def kv_int8_quant_ref(kv_bf16_bits: np.ndarray, group: int):
    """Rows [R, W] (bf16 bits) -> (codes uint8 [R, W], scale f32 [R, W/group],
    mn f32 [R, W/group]), every step an IEEE float32 operation."""
    from .bf16 import bf16_bits_to_f32
    x = bf16_bits_to_f32(np.asarray(kv_bf16_bits, np.uint16))
    if x.ndim != 2:
        raise ValueError("expected K or V rows [R, W]")
    r, w = x.shape
    _check_group(w, group)
    if not np.all(np.isfinite(x)):
        raise ValueError("inputs must be finite")
    g = x.reshape(r, w // group, group)
    # + 0 makes a zero extreme +0 (the min or max of +0 and -0 is either)
    mn = (g.min(axis=2) + np.float32(0.0)).astype(np.float32)
    mx = (g.max(axis=2) + np.float32(0.0)).astype(np.float32)
    rng_ = (mx - mn).astype(np.float32)
    scale = (rng_ / np.float32(255.0)).astype(np.float32)
    assert scale.dtype == np.float32
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        diff = (g - mn[:, :, None]).astype(np.float32)
        q = np.rint((diff / safe[:, :, None]).astype(np.float32))
    q = np.clip(np.where(scale[:, :, None] > 0, q, 0.0), 0, 255).astype(np.uint8)
    return q.reshape(r, w), scale, mn.astype(np.float32)


def kv_int8_dequant_ref(codes: np.ndarray, scale: np.ndarray, mn: np.ndarray,
                        group: int):
    """bf16 bits [R, W] of bf16(fl32(fl32(q * scale) + mn))."""
    q = np.asarray(codes, np.uint8)
    r, w = q.shape
    _check_group(w, group)
    s = np.repeat(np.asarray(scale, np.float32), group, axis=1)
    m = np.repeat(np.asarray(mn, np.float32), group, axis=1)
    prod = q.astype(np.float32) * s
    val = (prod + m).astype(np.float32)
    assert prod.dtype == np.float32 and val.dtype == np.float32
    return f64_to_bf16_bits(val.astype(np.float64))


def kv_int8_read_ref(codes, scale, mn, tail_bf16_bits, group: int):
    """The cache read: the dequantized history rows followed by the bf16
    residual rows, [R_hist + R_tail, W] bf16 bits."""
    hist = kv_int8_dequant_ref(codes, scale, mn, group)
    tail = np.asarray(tail_bf16_bits, np.uint16)
    if tail.ndim != 2 or tail.shape[1] != hist.shape[1]:
        raise ValueError("the tail must have the history's width")
    return np.concatenate([hist, tail], axis=0)
