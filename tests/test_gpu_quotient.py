"""Exhaustive GPU check of the quantizer's fast-path division: over every
(bf16 value, bf16 amax) pair whose scale takes the fast path, the codes equal
those of the IEEE float32 quotient (the helper in tests/hip compares the
library's own quantize8 fast path with its general path)."""

import ctypes
import os

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hip",
                   "libquotient_check.so")


def _expected():
    """Pairs and skipped amax values, from the same enumeration on the host
    (IEEE float32 division by 448 in numpy)."""
    pairs = skipped = 0
    for e in range(-53, 70):
        for mant in range(128):
            bits = (e + 127) << 7 | mant
            amax = np.array([bits << 16], np.uint32).view(np.float32)[0]
            s = amax / np.float32(448.0)
            if 2.0 ** -60 <= s <= 2.0 ** 60:
                pairs += bits + 1
            else:
                skipped += 1
    return pairs, skipped


def test_fast_path_codes_equal_ieee_codes_for_every_pair():
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} is missing: run __graft_entry__.build()")
    lib = ctypes.CDLL(LIB)
    fn = lib.fp8w8a8_test_quotient_check
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.POINTER(ctypes.c_ulonglong)]
    counts = (ctypes.c_ulonglong * 3)()
    assert fn(counts) == 0
    pairs, skipped = _expected()
    assert counts[0] == pairs == 266928097
    assert counts[2] == skipped
    assert counts[1] == 0, f"{counts[1]} code groups differ"
