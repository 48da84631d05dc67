"""Pins of the oracle's per-token / per-channel quantizer (CPU only).

Pinned to: hand-derived rows (tests/golden/quant_rows.txt); exact rational
rounding of the float32 division the oracle relies on; the half-ulp error
bound of round-to-nearest; the closed form "the amax element maps to +-448";
sign symmetry; exact power-of-two scale equivariance; zero rows.
"""

import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import (DECODE_TABLE, bf16_bits_to_f32, encode, quant_act_ref,
                    quant_rows_ref, quant_weight_ref)
from workloads import bf16_from_f64, c1_inputs, c5_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "quant_rows.txt")


def _parse_golden():
    cases, cur = [], {}
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, val = line.split(":", 1)
            items = [t.strip() for t in val.split(",")]
            if key == "row":
                cur = {"row": [float(eval(t, {"__builtins__": {}})) for t in items]}
            elif key == "scale":
                cur["scale"] = int(items[0], 16)
            elif key == "codes":
                cur["codes"] = [int(t, 16) for t in items]
                cases.append(cur)
    return cases


@pytest.mark.parametrize("case", _parse_golden())
def test_golden_rows(case):
    bits = bf16_from_f64(np.array([case["row"]], dtype=np.float64))
    # the golden values are all exactly representable in bfloat16
    assert np.array_equal(bf16_bits_to_f32(bits)[0].astype(np.float64),
                          np.array(case["row"]))
    q, s = quant_act_ref(bits)
    assert s.view(np.uint32)[0] == case["scale"]
    assert q[0].tolist() == case["codes"]
    qw, sw = quant_weight_ref(bits)           # same math along weight rows
    assert np.array_equal(qw, q) and np.array_equal(sw.view(np.uint32),
                                                    s.view(np.uint32))


def _round_fraction_to_f32(fr: Fraction) -> float:
    """Exact round-to-nearest-even of a rational to float32 (test helper)."""
    if fr == 0:
        return 0.0
    neg = fr < 0
    a = -fr if neg else fr
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -126)                       # below: fixed subnormal quantum
    quantum = Fraction(2) ** (e - 23)
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    v = float(fl * quantum)
    assert abs(v) <= float(np.finfo(np.float32).max)
    return -v if neg else v


def test_float32_division_is_correctly_rounded():
    """The oracle's quotient fl32(x/s) equals the exact rational, rounded."""
    rng = np.random.default_rng(7)
    xs = bf16_bits_to_f32(rng.integers(0, 0x7F80, 4000).astype(np.uint16))
    xs = np.concatenate([xs, -xs[:100]])
    ss = (2.0 ** rng.uniform(-140, 30, xs.size)).astype(np.float32)
    # keep quotients finite and within the range that matters
    q = xs / ss
    ok = np.isfinite(q) & (np.abs(q) < 1e30)
    for x, s, got in zip(xs[ok], ss[ok], q[ok]):
        want = _round_fraction_to_f32(Fraction(float(x)) / Fraction(float(s)))
        assert float(got) == want, (x, s)


def _ulp_e4m3(v: np.ndarray) -> np.ndarray:
    a = np.abs(v.astype(np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    return np.where(a < 2.0 ** -6, 2.0 ** -9, 2.0 ** (e - 3))


def _check_half_ulp(xbits):
    x = bf16_bits_to_f32(xbits).astype(np.float64)
    q, s = quant_act_ref(xbits)
    s64 = s.astype(np.float64)[:, None]
    deq = DECODE_TABLE[q] * s64
    quot = np.where(s64 > 0, x / np.where(s64 > 0, s64, 1), 0)
    bound = 0.5 * np.minimum(_ulp_e4m3(quot), 32.0) * s64 + 2.0 ** -23 * np.abs(x)
    assert np.all(np.abs(deq - x) <= bound)


def test_half_ulp_bound_c1():
    x, _ = c1_inputs()
    _check_half_ulp(x)


def test_half_ulp_bound_heavy_tail():
    x, _ = c5_inputs(0, m=64)
    _check_half_ulp(x)


def test_amax_maps_to_448():
    x, _ = c1_inputs()
    q, s = quant_act_ref(x)
    xf = bf16_bits_to_f32(x)
    arg = np.argmax(np.abs(xf), axis=1)
    top = q[np.arange(q.shape[0]), arg]
    neg = xf[np.arange(q.shape[0]), arg] < 0
    assert np.all(top == np.where(neg, 0xFE, 0x7E))
    # and nothing exceeds 448 in magnitude
    assert np.all((q & 0x7F) <= 0x7E)


def test_zero_rows_and_sign_symmetry():
    x, _ = c5_inputs(1, m=32)       # row 0 is all zero in this workload
    q, s = quant_act_ref(x)
    assert s[0] == 0 and np.all(q[0] == 0)
    neg = x ^ np.uint16(0x8000)
    qn, sn = quant_act_ref(neg)
    assert np.array_equal(qn, q ^ np.uint8(0x80))
    assert np.array_equal(sn.view(np.uint32), s.view(np.uint32))


@pytest.mark.parametrize("j", [-20, -3, 1, 5, 30])
def test_power_of_two_equivariance(j):
    rng = np.random.default_rng(11)
    x = bf16_from_f64(rng.standard_normal((6, 256)))
    q, s = quant_act_ref(x)
    # multiply by 2^j exactly by shifting the bf16 exponent field
    exp = ((x >> 7) & 0xFF).astype(np.int64)
    assert np.all((exp == 0) | ((exp + j > 0) & (exp + j < 255)))
    xs = np.where(exp == 0, x, (x.astype(np.int64) + (j << 7))).astype(np.uint16)
    assert np.array_equal(bf16_bits_to_f32(xs), bf16_bits_to_f32(x) * np.float32(2.0 ** j))
    q2, s2 = quant_act_ref(xs)
    assert np.array_equal(q2, q)
    assert np.array_equal(s2, s * np.float32(2.0 ** j))


def test_quant_rows_against_exact_brute_force():
    """Small rows: every code equals the exhaustive-search encoding of the
    exactly rounded quotient, computed with Fractions from scratch."""
    from oracle import encode_exact
    rng = np.random.default_rng(5)
    x = bf16_from_f64(rng.standard_normal((3, 40)) * np.array([[1e-3], [1.0], [1e3]]))
    q, s = quant_act_ref(x)
    xf = bf16_bits_to_f32(x)
    for r in range(3):
        amax = max(abs(Fraction(float(v))) for v in xf[r])
        s_exact = _round_fraction_to_f32(amax / 448)
        assert float(s[r]) == s_exact
        for c in range(40):
            quo = _round_fraction_to_f32(Fraction(float(xf[r, c])) / Fraction(s_exact))
            assert q[r, c] == encode_exact(quo)


def test_empty_and_shape_errors():
    q, s = quant_rows_ref(np.zeros((3, 0), np.float32))
    assert q.shape == (3, 0) and s.shape == (3,)
    q, s = quant_rows_ref(np.zeros((0, 8), np.float32))
    assert q.shape == (0, 8) and s.shape == (0,)
    with pytest.raises(ValueError):
        quant_rows_ref(np.array([[1.0, np.inf]], np.float32))
