"""E4M3 ("float8_e4m3fn") codec of the CPU oracle — test infrastructure only.

The pages name the storage type ``float8_e4m3fn`` (MOSS-VL quantization
README, "FP8-Dynamic" recipe) and describe it as 4 exponent bits and
3 mantissa bits (MOSS-VL-Realtime-FP8 article, section on why the 252
Linears use FP8 E4M3).  They give nothing more; the rest is the OCP 8-bit
floating point (OFP8) E4M3 definition that the ``fn`` name refers to:

* a code is ``s eeee mmm``; exponent bias 7;
* ``e == 0``: subnormal, value ``(-1)^s * m * 2^-9`` (includes +0 and -0);
* ``e > 0``: normal, value ``(-1)^s * (1 + m/8) * 2^(e-7)``;
* ``e == 15 and m == 7`` is NaN (codes 0x7F and 0xFF); there are no
  infinities, so ``s 1111 110`` = 448 is the largest finite magnitude.

Encoding (reading of the pages, which are silent on it): the code of the
finite E4M3 value nearest to ``v``; a tie goes to the code whose last bit is
0 (round half to even); magnitudes at or above 448 give 448 (saturation,
never NaN); the sign bit is copied from ``v``, so -0 and negative values that
round to zero give 0x80.  Codes are monotone in magnitude, which is why
"even code" and "even mantissa" coincide, also at the subnormal/normal
border (7.5 * 2^-9 is a tie between 0x07 and 0x08 and goes to 0x08).
"""

from fractions import Fraction
import math

import numpy as np

FINITE_MAX = 448.0


def decode(code: int) -> float:
    """Value of one E4M3 code, from its bit fields (NaN for 0x7F/0xFF)."""
    if not 0 <= code <= 255:
        raise ValueError("an E4M3 code is one byte")
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return math.nan
    if exp == 0:
        return sign * man * 2.0 ** -9
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


#: decode(c) for every byte c, in float64 (exact: every E4M3 value is dyadic
#: with at most 4 significant bits).
DECODE_TABLE = np.array([decode(c) for c in range(256)], dtype=np.float64)

#: the 127 non-negative finite values, indexed by their code 0x00..0x7E.
#: Increasing, since the codec is monotone on non-negative codes.
POSITIVE_VALUES = DECODE_TABLE[:0x7F].copy()


def _nearest_code_exact(mag: Fraction) -> int:
    """Brute force: scan all 127 non-negative codes, keep the nearest."""
    best_code, best_dist = None, None
    for code in range(0x7F):
        dist = abs(Fraction(POSITIVE_VALUES[code]) - mag)
        if best_dist is None or dist < best_dist or (
                dist == best_dist and code % 2 == 0):
            best_code, best_dist = code, dist
    return best_code


def encode_exact(v) -> int:
    """Encode one finite number (float or Fraction) by exhaustive search.

    Distances are compared in exact rational arithmetic over all 127
    candidate magnitudes, so this is the definition itself, written out.
    Slow; used to pin :func:`encode` on chosen values.
    """
    if isinstance(v, Fraction):
        negative = v < 0
        mag = abs(v)
    else:
        v = float(v)
        if math.isnan(v) or math.isinf(v):
            raise ValueError("only finite values have an E4M3 code here")
        negative = math.copysign(1.0, v) < 0  # -0.0 counts as negative
        mag = abs(Fraction(v))
    code = _nearest_code_exact(mag)
    return code | (0x80 if negative else 0)


def encode(v: np.ndarray) -> np.ndarray:
    """Encode an array of finite float32 values to E4M3 codes (uint8).

    Same definition as :func:`encode_exact`, vectorised: for each magnitude
    ``a`` find the two neighbouring table values ``lo <= a <= hi`` with a
    binary search, pick the nearer one, and on a tie the even code.  The
    comparison ``2a`` against ``lo + hi`` is exact in float64 (``a`` is a
    float32, ``lo`` and ``hi`` have 4 significant bits).
    """
    v = np.asarray(v, dtype=np.float32)
    if not np.all(np.isfinite(v)):
        raise ValueError("only finite values have an E4M3 code here")
    a = np.abs(v.astype(np.float64))
    hi_idx = np.searchsorted(POSITIVE_VALUES, a, side="left")
    hi_idx = np.minimum(hi_idx, 0x7E)          # saturate at 448
    lo_idx = np.maximum(hi_idx - 1, 0)
    lo = POSITIVE_VALUES[lo_idx]
    hi = POSITIVE_VALUES[hi_idx]
    twice = 2.0 * a
    mid = lo + hi
    pick_hi = (twice > mid) | ((twice == mid) & (hi_idx % 2 == 0))
    # a > 448: hi is clamped to 448 (0x7E) and lo is 416, so 2a > lo + hi
    # always picks 448: saturation needs no separate branch.
    # a == 0 exactly: hi_idx == 0 and lo_idx == 0, both give code 0.
    code = np.where(pick_hi, hi_idx, lo_idx).astype(np.uint8)
    sign = np.signbit(v).astype(np.uint8) << 7
    return (code | sign).astype(np.uint8)
