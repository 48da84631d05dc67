"""Pins of the oracle's RMSNorm -> per-token quantization (CPU only).

Pinned to: hand-derived rows (tests/golden/rmsnorm_rows.txt) that tell the
mean of squares from their sum, eps inside the root from outside, and the
two bfloat16 roundings of a BF16 norm from a single one; exact rational
brute force of both roundings on small rows; torch's own float64 ``rms_norm``
(a library routine for the unrounded normalization) and its bfloat16
multiply; closed forms (rows of +-1 or of one constant give +-gamma
exactly); exact power-of-two invariance at eps = 0; the zero row.
"""

import math
import os
import struct
from fractions import Fraction

import numpy as np
import pytest

from oracle import bf16_bits_to_f32, quant_act_ref
from oracle.norm import rmsnorm_quant_ref, rmsnorm_ref
from workloads import bf16_from_f64, norm_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "rmsnorm_rows.txt")


def _parse_golden():
    cases, cur = [], {}
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, val = (s.strip() for s in line.split(":", 1))
            items = [t.strip() for t in val.split(",")]
            if key in ("x", "gamma"):
                cur[key] = [float(t) for t in items]
            elif key == "eps":
                cur[key] = float(items[0])
            elif key in ("t", "y"):
                cur[key] = [int(t, 16) for t in items]
            elif key == "scale":
                cur[key] = int(items[0], 16)
            elif key == "codes":
                cur[key] = [int(t, 16) for t in items]
                cases.append(cur)
                cur = {}
    return cases


CASES = _parse_golden()


def test_golden_file_parsed():
    assert len(CASES) == 4


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"x{c['x']}-eps{c['eps']}")
def test_golden_rows(case):
    x = bf16_from_f64(np.array([case["x"]]))
    g = bf16_from_f64(np.array(case["gamma"]))
    # The fixture's decimals are exact bfloat16 values.
    assert np.array_equal(bf16_bits_to_f32(x)[0].astype(np.float64), case["x"])
    assert np.array_equal(bf16_bits_to_f32(g).astype(np.float64), case["gamma"])
    y, t = rmsnorm_ref(x, g, case["eps"])
    assert [int(b) for b in bf16_from_f64(t)[0]] == case["t"]
    assert [int(b) for b in y[0]] == case["y"]
    qx, sx, y2 = rmsnorm_quant_ref(x, g, case["eps"])
    assert np.array_equal(y2, y)
    assert int(sx.view(np.uint32)[0]) == case["scale"]
    assert [int(c) for c in qx[0]] == case["codes"]


# ---- exact rational brute force -------------------------------------------

def _bits_val(bits: int) -> Fraction:
    return Fraction(struct.unpack("<f", struct.pack("<I", (bits & 0xFFFF) << 16))[0])


def _round_frac(r: Fraction) -> int:
    """bfloat16 bits of the nearest value to the rational r (ties to even)."""
    if r == 0:
        return 0
    sign = 0x8000 if r < 0 else 0
    a = abs(r)
    e = math.floor(math.log2(a))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    assert e >= -126, "small rows only"
    q = a / Fraction(2) ** (e - 7)
    n = math.floor(q)
    fr = q - n
    if fr > Fraction(1, 2) or (fr == Fraction(1, 2) and n % 2 == 1):
        n += 1
    v = Fraction(n) * Fraction(2) ** (e - 7)
    bits = struct.unpack("<I", struct.pack("<f", float(v)))[0]
    assert bits & 0xFFFF == 0
    return sign | (bits >> 16)


def _round_root(num2: Fraction, sign: int) -> int:
    """bfloat16 bits of the nearest value to sign * sqrt(num2), num2 > 0,
    decided with exact comparisons of squares against the midpoints."""
    b = struct.unpack("<I", struct.pack("<f", math.sqrt(float(num2))))[0] >> 16
    while True:
        lo = (_bits_val(b - 1) + _bits_val(b)) / 2
        hi = (_bits_val(b) + _bits_val(b + 1)) / 2
        if num2 < lo * lo:
            b -= 1
        elif num2 > hi * hi:
            b += 1
        else:
            if (num2 == lo * lo or num2 == hi * hi) and b % 2 == 1:
                b += 1 if num2 == hi * hi else -1
            return sign | b


def test_brute_force_exact_rounding_small_rows():
    rng = np.random.default_rng(11)
    for k in (1, 2, 3, 8, 16):
        for eps in (0.0, 1e-6, 0.25):
            x = bf16_from_f64(rng.standard_normal((12, k)) * 3.0)
            g = bf16_from_f64(rng.standard_normal(k))
            y, t = rmsnorm_ref(x, g, eps)
            t_bits = bf16_from_f64(t)
            xf = bf16_bits_to_f32(x).astype(np.float64)
            gf = bf16_bits_to_f32(g).astype(np.float64)
            for m in range(x.shape[0]):
                ms = sum(Fraction(v) ** 2 for v in xf[m]) / k
                q = ms + Fraction(eps)
                for j in range(k):
                    xv = Fraction(xf[m, j])
                    if xv == 0:
                        continue
                    want_t = _round_root(xv * xv / q, 0x8000 if xv < 0 else 0)
                    assert int(t_bits[m, j]) == want_t, (k, eps, m, j)
                    want_y = _round_frac(Fraction(gf[j]) * _bits_val(want_t))
                    assert int(y[m, j]) == want_y, (k, eps, m, j)


# ---- library special case: torch's float64 rms_norm and bf16 multiply -------

def test_against_torch_rms_norm_and_bf16_product():
    torch = pytest.importorskip("torch")
    x, g = norm_inputs(8, 512, seed=3)
    eps = 1e-6
    y, t = rmsnorm_ref(x, g, eps)
    x64 = torch.from_numpy(bf16_bits_to_f32(x).astype(np.float64))
    ref = torch.nn.functional.rms_norm(x64, (x.shape[1],), eps=eps).numpy()
    np.testing.assert_allclose(t, ref, rtol=1e-13, atol=0)
    # Step 3 with torch's bfloat16 arithmetic on the rounded t.
    tb = torch.from_numpy(bf16_from_f64(t).astype(np.int16)).view(torch.bfloat16)
    gb = torch.from_numpy(g.astype(np.int16)).view(torch.bfloat16)
    yt = (gb[None, :] * tb).view(torch.int16).numpy().astype(np.uint16)
    assert np.array_equal(yt, y)


# ---- closed forms and invariants -----------------------------------------

def test_unit_rms_rows_give_signed_gamma():
    rng = np.random.default_rng(5)
    k = 64
    signs = rng.integers(0, 2, (6, k)).astype(np.uint16)
    x = (0x3F80 | (signs << 15)).astype(np.uint16)          # +-1.0
    g = bf16_from_f64(rng.standard_normal(k))
    y, t = rmsnorm_ref(x, g, 0.0)
    assert np.array_equal(y, (g[None, :] ^ (signs << 15)).astype(np.uint16))


def test_constant_rows_give_gamma():
    rng = np.random.default_rng(6)
    k = 48
    g = bf16_from_f64(rng.standard_normal(k))
    for c in (-3.0, 0.0078125, 1e10):
        x = bf16_from_f64(np.full((1, k), c))
        y, _ = rmsnorm_ref(x, g, 0.0)
        want = g ^ np.uint16(0x8000) if c < 0 else g
        assert np.array_equal(y[0], want)


@pytest.mark.parametrize("j", [-9, 5])
def test_power_of_two_invariance(j):
    x, g = norm_inputs(4, 256, seed=7)
    xs = (x.astype(np.int32) + (j << 7)).astype(np.uint16)   # x * 2^j, exact
    assert np.array_equal(bf16_bits_to_f32(xs).astype(np.float64),
                          bf16_bits_to_f32(x).astype(np.float64) * 2.0 ** j)
    assert np.array_equal(rmsnorm_ref(xs, g, 0.0)[0], rmsnorm_ref(x, g, 0.0)[0])


def test_eps_shrinks_magnitudes():
    x, g = norm_inputs(4, 128, seed=8)
    t0 = rmsnorm_ref(x, g, 0.0)[1]
    t1 = rmsnorm_ref(x, g, 0.5)[1]
    assert np.all(np.abs(t1) <= np.abs(t0))
    assert np.all(np.abs(t1) < np.abs(t0)) or np.all(x == 0)


def test_zero_rows_and_empty():
    g = bf16_from_f64(np.arange(1, 9, dtype=np.float64))
    x = np.zeros((2, 8), np.uint16)
    x[1, 3] = 0x8000                                          # a -0.0
    qx, sx, y = rmsnorm_quant_ref(x, g, 1e-6)
    assert np.all(sx == 0)
    assert int(y[1, 3]) == 0x8000 and int(qx[1, 3]) == 0x80   # sign kept
    assert np.all(np.delete(y.ravel(), 11) == 0)
    qx, sx, y = rmsnorm_quant_ref(np.zeros((0, 8), np.uint16), g, 1e-6)
    assert qx.shape == (0, 8) and sx.shape == (0,)


def test_quantization_of_the_norm_output():
    x, g = norm_inputs(16, 1024, seed=9)
    qx, sx, y = rmsnorm_quant_ref(x, g, 1e-6)
    q2, s2 = quant_act_ref(y)
    assert np.array_equal(qx, q2) and np.array_equal(sx, s2)
    # The amax element of each row encodes to +-448.
    yf = bf16_bits_to_f32(y)
    arg = np.argmax(np.abs(yf), axis=1)
    assert np.all((qx[np.arange(16), arg] & 0x7F) == 0x7E)
    # Scales are amax / 448 of the norm output, not of the input.
    assert np.allclose(sx, np.max(np.abs(yf), axis=1) / 448, rtol=2 ** -23)


def test_rejects_bad_arguments():
    x, g = norm_inputs(2, 16, seed=1)
    with pytest.raises(ValueError):
        rmsnorm_ref(x, g[:8], 1e-6)
    with pytest.raises(ValueError):
        rmsnorm_ref(x, g, -1.0)
