"""Pins of the oracle's SiLU-gated activation -> per-token quantization
(CPU only).

Pinned to: hand-derived rows (tests/golden/swiglu_rows.txt), one of which
separates the two bfloat16 roundings of a BF16 module from a single one;
scipy's logistic function (a library routine: silu(g) = g * expit(g)); the
exact rounding of silu to bfloat16 decided at 50 significant digits with
Python's decimal module; the identity silu(g) - silu(-g) = g; the limits
silu(g) -> g and silu(-g) -> -0 for large g; signed zeros.
"""

import math
import os
import struct
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

from oracle import bf16_bits_to_f32, quant_act_ref
from oracle.swiglu import silu_f64, swiglu_quant_ref, swiglu_ref
from workloads import bf16_from_f64

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "swiglu_rows.txt")


def _parse():
    cases, cur = [], {}
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, val = (t.strip() for t in line.split(":", 1))
            items = [t.strip() for t in val.split(",")]
            if key in ("g", "u"):
                cur[key] = [float(t) for t in items]
            elif key in ("s", "h", "codes"):
                cur[key] = [int(t, 16) for t in items]
            elif key == "scale":
                cur[key] = int(items[0], 16)
            if key == "codes":
                cases.append(cur)
                cur = {}
    return cases


CASES = _parse()


def test_golden_file_parsed():
    assert len(CASES) == 2


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"g{c['g']}")
def test_golden_rows(case):
    g = bf16_from_f64(np.array([case["g"]]))
    u = bf16_from_f64(np.array([case["u"]]))
    assert np.array_equal(bf16_bits_to_f32(g)[0].astype(np.float64), case["g"])
    assert np.array_equal(bf16_bits_to_f32(u)[0].astype(np.float64), case["u"])
    h, s, _ = swiglu_ref(g, u)
    assert [int(b) for b in s[0]] == case["s"]
    assert [int(b) for b in h[0]] == case["h"]
    qh, sh, h2 = swiglu_quant_ref(g, u)
    assert np.array_equal(h2, h)
    assert int(sh.view(np.uint32)[0]) == case["scale"]
    assert [int(c) for c in qh[0]] == case["codes"]


def test_against_scipy_expit():
    special = pytest.importorskip("scipy.special")
    rng = np.random.default_rng(3)
    g = bf16_bits_to_f32(bf16_from_f64(rng.standard_normal(4000) * 6)).astype(np.float64)
    np.testing.assert_allclose(silu_f64(g), g * special.expit(g), rtol=4e-16, atol=0)


def _bf16_round_fraction(r: Fraction) -> int:
    if r == 0:
        return 0
    sign = 0x8000 if r < 0 else 0
    a = abs(r)
    e = math.floor(math.log2(a))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    if e < -126:                      # bfloat16 subnormal spacing
        e = -126
    q = a / Fraction(2) ** (e - 7)
    n = math.floor(q)
    fr = q - n
    if fr > Fraction(1, 2) or (fr == Fraction(1, 2) and n % 2 == 1):
        n += 1
    v = float(Fraction(n) * Fraction(2) ** (e - 7))
    return sign | (struct.unpack("<I", struct.pack("<f", v))[0] >> 16)


def test_rounding_of_silu_decided_at_50_digits():
    getcontext().prec = 50
    rng = np.random.default_rng(4)
    g_bits = bf16_from_f64(np.concatenate([rng.standard_normal(300) * 4,
                                           rng.uniform(-90, 30, 100)]))
    _, s_bits, _ = swiglu_ref(g_bits, np.full_like(g_bits, 0x3F80))
    for gb, sb in zip(g_bits, s_bits):
        g = Decimal(float(bf16_bits_to_f32(np.array([gb]))[0]))
        silu = g / (1 + (-g).exp())
        assert _bf16_round_fraction(Fraction(silu)) == int(sb), float(g)


def test_odd_part_identity():
    rng = np.random.default_rng(5)
    g = rng.standard_normal(1000) * 8
    np.testing.assert_allclose(silu_f64(g) - silu_f64(-g), g, rtol=0, atol=1e-14 * 8)


def test_limits_and_signed_zeros():
    big = bf16_from_f64(np.array([8.0, 9.5, 100.0, 3.0e4, 1.0e30]))
    _, s, _ = swiglu_ref(big, np.full_like(big, 0x3F80))
    assert np.array_equal(s, big)                      # silu(g) rounds to g
    neg = bf16_from_f64(np.array([-110.0, -1.0e3, -3.0e38]))
    _, s, _ = swiglu_ref(neg, np.full_like(neg, 0x3F80))
    assert np.all(s == 0x8000)                         # -0
    z = np.array([0x0000, 0x8000, 0x0000, 0x8000], np.uint16)
    u = np.array([0x3F80, 0x3F80, 0xBF80, 0xBF80], np.uint16)   # +1, +1, -1, -1
    h, s, _ = swiglu_ref(z, u)
    assert list(s) == [0x0000, 0x8000, 0x0000, 0x8000]
    assert list(h) == [0x0000, 0x8000, 0x8000, 0x0000]


def test_quantization_of_the_activation():
    rng = np.random.default_rng(6)
    g = bf16_from_f64(rng.standard_normal((8, 512)) * 3)
    u = bf16_from_f64(rng.standard_normal((8, 512)) * 3)
    qh, sh, h = swiglu_quant_ref(g, u)
    q2, s2 = quant_act_ref(h)
    assert np.array_equal(qh, q2) and np.array_equal(sh, s2)
    hf = bf16_bits_to_f32(h)
    arg = np.argmax(np.abs(hf), axis=1)
    assert np.all((qh[np.arange(8), arg] & 0x7F) == 0x7E)


def test_rejects_bad_arguments():
    a = np.zeros((2, 8), np.uint16)
    with pytest.raises(ValueError):
        swiglu_ref(a, a[:, :4])
    b = a.copy()
    b[0, 0] = 0x7F80                                   # +inf
    with pytest.raises(ValueError):
        swiglu_ref(b, a)
