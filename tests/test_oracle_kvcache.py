"""Pins of the oracle's FP8 E4M3 KV-cache codec (CPU only).

Pinned to: a hand-derived row (tests/golden/kv_fp8_rows.txt) with a tie to
the even mantissa, a signed zero and a group whose scale is inexact; the
reduction to the per-token quantizer when the group is the whole row;
reading back every code under power-of-two scales (exact values: pins the
decode table and the scale's use as a multiplier); the float32 product and
the bf16 rounding against exact rational arithmetic for every code under
random scales; the round-trip error bound (half an E4M3 step plus the bf16
rounding).
"""

import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import DECODE_TABLE, bf16_bits_to_f32, quant_act_ref
from oracle.kvcache import kv_fp8_dequant_ref, kv_fp8_quant_ref
from workloads import bf16_from_f64

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kv_fp8_rows.txt")


def _golden():
    d = {}
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, val = (t.strip() for t in line.split(":", 1))
            d[key] = [t.strip() for t in val.split(",")]
    return d


def test_golden_row():
    g = _golden()
    x = bf16_from_f64(np.array([[float(t) for t in g["x"]]]))
    assert x[0, 4] == 0x8000
    group = int(g["group"][0])
    codes, scales = kv_fp8_quant_ref(x, group)
    assert [int(c) for c in codes[0]] == [int(t, 16) for t in g["codes"]]
    assert [int(v) for v in scales[0].view(np.uint32)] == [int(t, 16) for t in g["scales"]]
    back = kv_fp8_dequant_ref(codes, scales, group)
    assert [int(b) for b in back[0]] == [int(t, 16) for t in g["back"]]


def test_whole_row_group_is_the_per_token_quantizer():
    rng = np.random.default_rng(1)
    x = bf16_from_f64(rng.standard_normal((9, 1024)) * 3)
    c1, s1 = kv_fp8_quant_ref(x, 1024)
    c2, s2 = quant_act_ref(x)
    assert np.array_equal(c1, c2) and np.array_equal(s1[:, 0], s2)


def test_groups_are_independent_rows():
    rng = np.random.default_rng(2)
    x = bf16_from_f64(rng.standard_normal((3, 512)) * np.array([1e-3, 1.0, 1e3])[:, None])
    c, s = kv_fp8_quant_ref(x, 128)
    for i in range(3):
        for j in range(4):
            cq, sq = quant_act_ref(x[i:i + 1, 128 * j:128 * (j + 1)])
            assert np.array_equal(c[i, 128 * j:128 * (j + 1)], cq[0])
            assert s[i, j] == sq[0]


def test_read_back_every_code_under_power_of_two_scales():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    for e in (-20, -3, 0, 5, 30):
        back = kv_fp8_dequant_ref(codes[None, :], np.full((1, 1), 2.0 ** e, np.float32),
                                  codes.size)
        want = DECODE_TABLE[codes] * 2.0 ** e         # exact: <= 4 significant bits
        got = bf16_bits_to_f32(back[0]).astype(np.float64)
        assert np.array_equal(got, want)
        assert np.array_equal(np.signbit(got), np.signbit(want))


def _f32_round(q: Fraction) -> Fraction:
    """Nearest float32 to q (ties to even), exact rational arithmetic, for
    normal results."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    step = Fraction(2) ** (e - 23)
    n, rem = divmod(a, step)
    n = int(n)
    if rem * 2 > step or (rem * 2 == step and n % 2 == 1):
        n += 1
    return sign * n * step


def test_float32_product_then_bf16_against_exact_arithmetic():
    rng = np.random.default_rng(3)
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    scales = (rng.uniform(0.5, 2.0, 6) * 2.0 ** rng.integers(-40, 40, 6)).astype(np.float32)
    for sc in scales:
        back = kv_fp8_dequant_ref(codes[None, :], np.array([[sc]], np.float32), codes.size)
        for c, b in zip(codes, back[0]):
            exact = Fraction(float(DECODE_TABLE[c])) * Fraction(float(sc))
            p32 = _f32_round(exact)
            want = bf16_from_f64(np.array([float(p32)]))[0]
            if p32 == 0:
                want = 0x8000 if c & 0x80 else 0
            assert int(b) == int(want), (hex(c), float(sc))


def test_round_trip_error_bound():
    rng = np.random.default_rng(4)
    x = bf16_from_f64(rng.standard_normal((16, 1024)) * 4)
    c, s = kv_fp8_quant_ref(x, 128)
    back = bf16_bits_to_f32(kv_fp8_dequant_ref(c, s, 128)).astype(np.float64)
    xf = bf16_bits_to_f32(x).astype(np.float64)
    sg = np.repeat(s.astype(np.float64), 128, axis=1)
    # half an E4M3 step (2^-4 relative for normals, 2^-10 s for subnormals),
    # then the bf16 rounding of the read-back value (half a bf16 step: at
    # most 2^-8 relative, just above a power of two)
    bound = np.maximum(2.0 ** -4 * np.abs(xf), 2.0 ** -10 * sg) * (1 + 2.0 ** -8) \
        + 2.0 ** -8 * np.abs(back) + 1e-30
    assert np.all(np.abs(back - xf) <= bound)


def test_rejects_bad_groups():
    x = np.zeros((2, 96), np.uint16)
    with pytest.raises(ValueError):
        kv_fp8_quant_ref(x, 64)
    c = np.zeros((2, 96), np.uint8)
    with pytest.raises(ValueError):
        kv_fp8_dequant_ref(c, np.zeros((2, 2), np.float32), 32)


# ---- INT8 group-wise cache with a BF16 residual window ----------------------

from oracle.kvcache import kv_int8_dequant_ref, kv_int8_quant_ref, kv_int8_read_ref

GOLDEN8 = os.path.join(os.path.dirname(__file__), "golden", "kv_int8_rows.txt")


def test_int8_golden_row():
    g = {}
    with open(GOLDEN8) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = (t.strip() for t in line.split(":", 1))
                g[k] = [t.strip() for t in v.split(",")]
    x = bf16_from_f64(np.array([[float(t) for t in g["x"]]]))
    group = int(g["group"][0])
    q, s, m = kv_int8_quant_ref(x, group)
    assert [int(c) for c in q[0]] == [int(t, 16) for t in g["codes"]]
    assert [int(v) for v in s[0].view(np.uint32)] == [int(t, 16) for t in g["scales"]]
    assert [int(v) for v in m[0].view(np.uint32)] == [int(t, 16) for t in g["mins"]]
    back = kv_int8_dequant_ref(q, s, m, group)
    assert [int(b) for b in back[0]] == [int(t, 16) for t in g["back"]]


def test_int8_extremes_map_to_0_and_255_and_constant_groups():
    rng = np.random.default_rng(11)
    x = bf16_from_f64(rng.standard_normal((20, 512)) * 10 ** rng.uniform(-3, 3, (20, 1)))
    x[3, 64:128] = x[3, 64]                                # a constant group
    q, s, m = kv_int8_quant_ref(x, 64)
    xf = bf16_bits_to_f32(x).reshape(20, 8, 64)
    qg = q.reshape(20, 8, 64)
    lo = np.argmin(xf, axis=2)
    hi = np.argmax(xf, axis=2)
    for i in range(20):
        for j in range(8):
            if s[i, j] == 0:
                assert np.all(qg[i, j] == 0)
                continue
            assert qg[i, j, lo[i, j]] == 0 and qg[i, j, hi[i, j]] == 255
    assert s[3, 1] == 0
    back = bf16_bits_to_f32(kv_int8_dequant_ref(q, s, m, 64)).reshape(20, 8, 64)
    assert np.all(back[3, 1] == xf[3, 1, 0])               # constant groups read back exactly


def _f32(q: Fraction) -> Fraction:
    return _f32_round(q)


def test_int8_steps_against_exact_arithmetic():
    """Every float32 step of the quantizer, decided in exact rational
    arithmetic, on small groups of random bf16 values."""
    rng = np.random.default_rng(12)
    x = bf16_from_f64(rng.standard_normal((40, 16)) * 5)
    q, s, m = kv_int8_quant_ref(x, 8)
    xf = bf16_bits_to_f32(x).astype(np.float64)
    for i in range(40):
        for j in range(2):
            grp = [Fraction(v) for v in xf[i, 8 * j:8 * (j + 1)]]
            mn, mx = min(grp), max(grp)
            sc = _f32(_f32(mx - mn) / 255)
            assert Fraction(float(s[i, j])) == sc and Fraction(float(m[i, j])) == mn
            for k, v in enumerate(grp):
                quo = _f32(_f32(v - mn) / sc)
                n = int(quo)                               # floor for quo >= 0
                frac = quo - n
                if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and n % 2 == 1):
                    n += 1
                assert int(q[i, 8 * j + k]) == min(max(n, 0), 255)


def test_int8_round_trip_error_bound():
    rng = np.random.default_rng(13)
    x = bf16_from_f64(rng.standard_normal((32, 1024)) * 3)
    q, s, m = kv_int8_quant_ref(x, 64)
    back = bf16_bits_to_f32(kv_int8_dequant_ref(q, s, m, 64)).astype(np.float64)
    xf = bf16_bits_to_f32(x).astype(np.float64)
    sg = np.repeat(s.astype(np.float64), 64, axis=1)
    # half a step, a few float32 roundings of values up to the group's range,
    # then the bf16 rounding of the read-back value
    rngw = 255 * sg
    bound = 0.5 * sg * (1 + 2.0 ** -20) + 4 * 2.0 ** -24 * rngw + 2.0 ** -8 * np.abs(back)
    assert np.all(np.abs(back - xf) <= bound + 1e-30)


def test_int8_read_is_history_then_tail():
    rng = np.random.default_rng(14)
    hist = bf16_from_f64(rng.standard_normal((300, 256)))
    tail = bf16_from_f64(rng.standard_normal((100, 256)))
    q, s, m = kv_int8_quant_ref(hist, 64)
    out = kv_int8_read_ref(q, s, m, tail, 64)
    assert out.shape == (400, 256)
    assert np.array_equal(out[:300], kv_int8_dequant_ref(q, s, m, 64))
    assert np.array_equal(out[300:], tail)
