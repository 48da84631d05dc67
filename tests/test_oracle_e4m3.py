"""Pins of the oracle's E4M3 codec (CPU only).

The codec is pinned to things other than itself: closed forms of the bit
fields, hand-derived golden codes (tests/golden/e4m3_codes.txt), exhaustive
search in exact rational arithmetic, and torch's independent CPU
``float8_e4m3fn`` cast (which rounds to nearest-even but returns NaN above
464, so it is compared after clamping to +-448).
"""

import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import DECODE_TABLE, POSITIVE_VALUES, decode, encode, encode_exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_codes.txt")


def test_decode_closed_form():
    assert DECODE_TABLE[0x7E] == 448.0
    assert DECODE_TABLE[0xFE] == -448.0
    assert DECODE_TABLE[0x08] == 2.0 ** -6
    assert DECODE_TABLE[0x01] == 2.0 ** -9
    assert DECODE_TABLE[0x07] == 7 * 2.0 ** -9
    assert DECODE_TABLE[0x38] == 1.0
    assert DECODE_TABLE[0x00] == 0.0 and not math.copysign(1, DECODE_TABLE[0x00]) < 0
    assert DECODE_TABLE[0x80] == 0.0 and math.copysign(1, DECODE_TABLE[0x80]) < 0
    nan_codes = [c for c in range(256) if math.isnan(DECODE_TABLE[c])]
    assert nan_codes == [0x7F, 0xFF]
    pos = DECODE_TABLE[1:0x7F]
    assert len(pos) == 126 and np.all(np.diff(pos) > 0)
    for c in range(0x7F):
        assert DECODE_TABLE[c | 0x80] == -DECODE_TABLE[c]
    # every value has at most 4 significant bits
    for c in range(1, 0x7F):
        f = Fraction(DECODE_TABLE[c])
        while f.denominator > 1 and f.numerator % 2 == 0:
            f /= 2
        n = f.numerator
        while n % 2 == 0:
            n //= 2
        assert n < 16


def test_decode_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    t = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    same = (t == DECODE_TABLE) | (np.isnan(t) & np.isnan(DECODE_TABLE))
    assert same.all()
    fin = ~np.isnan(DECODE_TABLE)
    assert np.array_equal(np.signbit(t[fin]), np.signbit(DECODE_TABLE[fin]))


def _golden_lines():
    out = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            expr, code = line.split()
            out.append((float(eval(expr, {"__builtins__": {}})), int(code, 16)))
    return out


@pytest.mark.parametrize("value,code", _golden_lines())
def test_golden_codes(value, code):
    v32 = np.float32(value)
    assert encode(np.array([v32]))[0] == code
    assert encode_exact(float(v32)) == code


def test_roundtrip_all_codes():
    finite = [c for c in range(256) if c not in (0x7F, 0xFF)]
    vals = np.array([decode(c) for c in finite], dtype=np.float32)
    assert list(encode(vals)) == finite
    assert [encode_exact(float(v)) for v in vals] == finite


def _midpoint_neighbourhood(ulps=3):
    """float32 values within a few ulps of every rounding boundary."""
    mids = (POSITIVE_VALUES[:-1] + POSITIVE_VALUES[1:]) / 2
    mids = np.concatenate([mids, POSITIVE_VALUES, [464.0, 480.0]])
    bits = mids.astype(np.float32).view(np.int32)
    out = [(bits + d).view(np.float32) for d in range(-ulps, ulps + 1)]
    v = np.concatenate(out)
    v = v[np.isfinite(v) & (v >= 0)]
    return np.concatenate([v, -v])


def test_encode_matches_exhaustive_search():
    rng = np.random.default_rng(1234)
    # random bf16 patterns whose magnitude spans the whole e4m3 range
    bf = rng.integers(0, 1 << 16, size=2500).astype(np.uint16)
    bf_vals = (bf.astype(np.uint32) << 16).view(np.float32)
    bf_vals = bf_vals[np.isfinite(bf_vals)]
    mag = rng.uniform(-13, 9.5, size=1500)
    logu = (np.sign(rng.standard_normal(1500)) * 2.0 ** mag).astype(np.float32)
    vals = np.concatenate([bf_vals, logu, _midpoint_neighbourhood()])
    fast = encode(vals)
    exact = np.array([encode_exact(float(v)) for v in vals], dtype=np.uint8)
    bad = np.nonzero(fast != exact)[0]
    assert bad.size == 0, [(float(vals[i]), fast[i], exact[i]) for i in bad[:5]]


def test_encode_exact_on_rationals():
    # exact ties given as fractions (no float rounding on the way in)
    assert encode_exact(Fraction(17, 16)) == 0x38
    assert encode_exact(Fraction(19, 16)) == 0x3A
    assert encode_exact(Fraction(15, 1024)) == 0x08      # 7.5 * 2^-9
    assert encode_exact(-Fraction(1, 1024)) == 0x80


def _torch_ref(v: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.clip(v, -448.0, 448.0).astype(np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_encode_matches_torch_all_bf16():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = (bits.astype(np.uint32) << 16).view(np.float32)
    v = v[np.isfinite(v)]
    assert np.array_equal(encode(v), _torch_ref(v))


def test_encode_matches_torch_dense_float32():
    # every 11th float32 bit pattern with magnitude in [2^-12, 2^9], both signs,
    # plus every pattern near a rounding boundary and every tiny subnormal
    lo = np.float32(2.0 ** -12).view(np.uint32)
    hi = np.float32(2.0 ** 9).view(np.uint32)
    pat = np.arange(lo, hi, 11, dtype=np.uint32)
    v = pat.view(np.float32)
    v = np.concatenate([v, -v, _midpoint_neighbourhood(16),
                        np.arange(0, 5000, dtype=np.uint32).view(np.float32)])
    for chunk in np.array_split(v, 8):
        assert np.array_equal(encode(chunk), _torch_ref(chunk))


def test_encode_rejects_non_finite():
    with pytest.raises(ValueError):
        encode(np.array([np.nan], dtype=np.float32))
    with pytest.raises(ValueError):
        encode_exact(math.inf)
