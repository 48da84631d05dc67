"""Pins of the oracle's matmul, epilogue and pass criteria (CPU only).

Pinned to: brute force in exact rational arithmetic on small non-square
problems (so a transposed operand, a swapped scale or a dropped term
fails), one-hot weights that pick single products, the bound
|acc| <= 448^2 K, linearity in the weight rows, and the bfloat16 rounding of
the report path against torch's CPU cast.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import (DECODE_TABLE, bf16_bits_to_f32, check_close, close_report,
                    f64_to_bf16_bits, linear_ref, quant_act_ref,
                    quant_linear_ref, quant_weight_ref)
from workloads import bf16_from_f64

FINITE_CODES = np.array([c for c in range(256) if c not in (0x7F, 0xFF)],
                        dtype=np.uint8)


def _random_codes(rng, shape):
    return rng.choice(FINITE_CODES, size=shape).astype(np.uint8)


@pytest.mark.parametrize("m,n,k", [(4, 8, 8), (3, 5, 7), (1, 6, 2), (5, 1, 9)])
def test_brute_force_fractions(m, n, k):
    rng = np.random.default_rng(m * 100 + n * 10 + k)
    qx, qw = _random_codes(rng, (m, k)), _random_codes(rng, (n, k))
    sx = (2.0 ** rng.uniform(-8, 8, m)).astype(np.float32)
    sw = (2.0 ** rng.uniform(-8, 8, n)).astype(np.float32)
    y = linear_ref(qx, sx, qw, sw)
    assert y.shape == (m, n)
    for i in range(m):
        for j in range(n):
            acc = sum(Fraction(DECODE_TABLE[qx[i, t]]) * Fraction(DECODE_TABLE[qw[j, t]])
                      for t in range(k))
            exact = acc * Fraction(float(sx[i])) * Fraction(float(sw[j]))
            if exact == 0:
                assert y[i, j] == 0
            else:
                assert abs(Fraction(float(y[i, j])) - exact) <= abs(exact) * Fraction(1, 2 ** 51)


def test_unit_scales_exact_sum():
    rng = np.random.default_rng(3)
    qx, qw = _random_codes(rng, (4, 8)), _random_codes(rng, (8, 8))
    y = linear_ref(qx, np.ones(4, np.float32), qw, np.ones(8, np.float32))
    for i in range(4):
        for j in range(8):
            acc = sum(Fraction(DECODE_TABLE[qx[i, t]]) * Fraction(DECODE_TABLE[qw[j, t]])
                      for t in range(8))
            assert Fraction(float(y[i, j])) == acc   # exact at this size


def test_one_hot_weights_pick_single_products():
    rng = np.random.default_rng(9)
    m, n, k = 5, 12, 16
    qx = _random_codes(rng, (m, k))
    perm = rng.permutation(k)[:n]
    qw = np.zeros((n, k), np.uint8)
    qw[np.arange(n), perm] = 0x38                       # 1.0
    sx = rng.uniform(0.5, 2, m).astype(np.float32)
    sw = rng.uniform(0.5, 2, n).astype(np.float32)
    y = linear_ref(qx, sx, qw, sw)
    want = (DECODE_TABLE[qx[:, perm]] * sx.astype(np.float64)[:, None]
            * sw.astype(np.float64)[None, :])
    assert np.array_equal(y, want)


def test_accumulator_bound_and_linearity():
    rng = np.random.default_rng(4)
    k = 64
    qx = np.full((2, k), 0x7E, np.uint8)
    qx[1] = 0xFE
    qw = np.full((3, k), 0x7E, np.uint8)
    y = linear_ref(qx, np.ones(2, np.float32), qw, np.ones(3, np.float32))
    assert np.all(y[0] == 448.0 ** 2 * k) and np.all(y[1] == -(448.0 ** 2) * k)
    qx = _random_codes(rng, (3, k))
    qa, qb = _random_codes(rng, (1, k)), _random_codes(rng, (1, k))
    one = np.ones(1, np.float32)
    ya = linear_ref(qx, np.ones(3, np.float32), qa, one)
    yb = linear_ref(qx, np.ones(3, np.float32), qb, one)
    yab = linear_ref(qx, np.ones(3, np.float32), np.concatenate([qa, qb]),
                     np.ones(2, np.float32))
    assert np.array_equal(yab, np.concatenate([ya, yb], axis=1))


def test_quant_linear_close_to_unquantized():
    """FP8_DYNAMIC result tracks the unquantized fp64 product (loose bound)."""
    rng = np.random.default_rng(2)
    x = bf16_from_f64(rng.standard_normal((8, 512)))
    w = bf16_from_f64(rng.standard_normal((32, 512)) * 0.02)
    qw, sw = quant_weight_ref(w)
    y, qx, sx = quant_linear_ref(x, qw, sw)
    exact = bf16_bits_to_f32(x).astype(np.float64) @ bf16_bits_to_f32(w).astype(np.float64).T
    rel = np.linalg.norm(y - exact) / np.linalg.norm(exact)
    assert rel < 0.06                 # e4m3 has 3 mantissa bits: ~2-3 % per factor
    assert np.array_equal(qx, quant_act_ref(x)[0])


def test_bf16_report_rounding_matches_torch():
    rng = np.random.default_rng(6)
    v = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.uniform(-40, 38, 20000),
                        [0.0, -0.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8]])
    # torch rounds float32 -> bf16; feed values exact in float32 to avoid
    # double rounding in the comparison
    v32 = v.astype(np.float32).astype(np.float64)
    want = torch.from_numpy(v32.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f64_to_bf16_bits(v32), want)


def test_check_close_plants():
    rng = np.random.default_rng(8)
    y64 = rng.standard_normal((4, 64))
    y64[2] = 0.0
    good = f64_to_bf16_bits(y64)
    check_close(good, y64)
    bad = bf16_from_f64(y64 * (1 + 0.03))           # 3 % off everywhere
    with pytest.raises(AssertionError):
        check_close(bad, y64)
    one_bad = good.copy()
    one_bad[1, 5] = bf16_from_f64(np.array([y64[1, 5] * 1.05 + 0.1]))[0]
    with pytest.raises(AssertionError):
        check_close(one_bad, y64)
    nonzero_row = good.copy()
    nonzero_row[2, 0] = bf16_from_f64(np.array([1e-30]))[0]
    with pytest.raises(AssertionError):
        check_close(nonzero_row, y64)
    nan = good.copy()
    nan[0, 0] = 0x7FC0
    with pytest.raises(AssertionError):
        check_close(nan, y64)
    assert close_report(good, y64)["frac_bf16_equal"] == 1.0
    # A small element (1 % of its row's RMS) off by 0.5 % of the row RMS,
    # i.e. 50 % of itself: within 1e-2 x the row RMS (the floor of 1.0 it
    # replaces), but not within 1e-2 x 2^-3 of it.
    small = y64.copy()
    rms1 = np.sqrt(np.mean(y64[1] ** 2))
    small[1, 7] = 0.01 * rms1
    off = f64_to_bf16_bits(small)
    off[1, 7] = bf16_from_f64(np.array([small[1, 7] + 0.005 * rms1]))[0]
    err = abs(float(bf16_bits_to_f32(off[1:2, 7:8])[0, 0]) - small[1, 7])
    rms_small = np.sqrt(np.mean(small[1] ** 2))
    assert 1e-2 * 2.0 ** -3 * rms_small < err < 1e-2 * rms_small
    with pytest.raises(AssertionError):
        check_close(off, small)
    # ... while an error of 1e-3 of the row RMS on it passes.
    ok = f64_to_bf16_bits(small)
    ok[1, 7] = bf16_from_f64(np.array([small[1, 7] + 0.001 * rms1]))[0]
    check_close(ok, small)
