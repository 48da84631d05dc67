"""bfloat16 helpers of the CPU oracle — test infrastructure only.

BF16 is the precision of everything the pages keep unquantized and the
dtype the checkpoint is loaded in (MOSS-VL quantization README, the
``precision="bfloat16"`` argument of the FP8-Dynamic one-shot call).  A
bfloat16 is the upper 16 bits of an IEEE float32: 1 sign, 8 exponent,
7 stored mantissa bits.
"""

import numpy as np


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening: place the 16 bits above 16 zero bits of a float32."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def f64_to_bf16_bits(y: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16, ties to even (one rounding).

    Written from the format: a normal bfloat16 has 8 significant bits, so
    ``y = f * 2^e`` with ``0.5 <= |f| < 1`` rounds to ``rint(f * 2^8) * 2^(e-8)``
    (``numpy.rint`` rounds half to even); below 2^-126 the spacing is fixed at
    2^-133; results above the largest finite value become infinities.  Used
    only to report how many outputs are bit-equal; the pass criterion uses the
    float64 value itself.
    """
    y = np.asarray(y, dtype=np.float64)
    f, e = np.frexp(y)
    r = np.ldexp(np.rint(np.ldexp(f, 8)), e - 8)
    tiny = np.abs(y) < 2.0 ** -126
    r = np.where(tiny, np.rint(y * 2.0 ** 133) * 2.0 ** -133, r)
    max_bf16 = (2.0 - 2.0 ** -7) * 2.0 ** 127
    r = np.where(np.abs(r) > max_bf16, np.copysign(np.inf, y), r)
    # Now r is exactly representable in bfloat16, hence in float32.
    r32 = r.astype(np.float32)
    return (r32.view(np.uint32) >> 16).astype(np.uint16)
