"""The seeded generators: determinism, shapes and the stated structure."""

import numpy as np

from oracle import bf16_bits_to_f32
from workloads import LAYER_SHAPES, c1_inputs, c2_inputs, c3_inputs, c5_inputs
from workloads.generators import bf16_from_f64, c5_rows


def test_layer_shapes():
    assert [(n, k) for _, n, k in LAYER_SHAPES] == [
        (4096, 4096), (1024, 4096), (1024, 4096), (4096, 4096),
        (12288, 4096), (12288, 4096), (4096, 12288)]
    assert sum(n * k for _, n, k in LAYER_SHAPES) == 192_937_984


def test_c1_deterministic_and_shaped():
    x1, w1 = c1_inputs()
    x2, w2 = c1_inputs()
    assert x1.shape == (16, 4096) and w1.shape == (4096, 4096)
    assert x1.dtype == np.uint16 and np.array_equal(x1, x2) and np.array_equal(w1, w2)
    xf = bf16_bits_to_f32(x1)
    big = np.abs(xf) > 6.0
    assert 0.005 < big.mean() < 0.015            # the 1 % x20 outliers
    wf = bf16_bits_to_f32(w1)
    assert abs(float(wf.std()) - 0.02) < 0.001


def test_c2_c3_seeds_differ_per_linear():
    xa, _ = c2_inputs(4, 0)
    xb, _ = c2_inputs(4, 1)
    assert xa.shape == (4, 4096) and not np.array_equal(xa, xb)
    x, w = c3_inputs(6, m=8)
    assert x.shape == (8, 12288) and w.shape == (4096, 12288)


def test_c5_special_rows():
    m = 2048
    zero, big, heavy = c5_rows(m)
    assert zero[0] == 0 and len(zero) == len(big) == len(heavy) == 3
    assert not set(zero) & set(big) and not set(big) & set(heavy)
    x, _ = c5_inputs(1, m=m)
    xf = bf16_bits_to_f32(x)
    assert np.all(xf[zero] == 0)
    assert np.all(np.abs(xf[big]).max(axis=1) > 1e4)
    for r in heavy:
        amax = np.abs(xf[r]).max()
        assert np.mean(np.abs(xf[r]) == amax) > 0.05


def test_bf16_rounding_is_nearest_even():
    v = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.5, 0.0], np.float64)
    bits = bf16_from_f64(v)
    assert bits.tolist() == [0x3F80, 0x3F82, 0xC020, 0x0000]
