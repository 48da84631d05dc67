"""The grouped one-token call (fp8w8a8_quant_linear_group_m1): several
independent FP8_DYNAMIC Linears at M = 1 in one launch must give, item by
item, the bits of fp8w8a8_quant_linear on each alone, and be within the
tolerance of the oracle.  Cases: the decode layer's 7 Linears (K = 4096 and
12288), ragged shapes (N = 16, K not a multiple of the 2 KB step), and
items of every K class in one launch."""

import numpy as np
import pytest
import torch

import fp8_w8a8_dynamic_amd as fq
import oracle
from oracle import check_bytes, check_close
from tests.gpu_util import host_bits, to_dev_bf16
from workloads import LAYER_SHAPES, bf16_from_f64, c2_inputs

pytestmark = pytest.mark.gpu


def _check_group(xs_bits, ws_bits, what, monkeypatch):
    """Grouped against each item alone through the one-token kernel (taken
    for every K here through the test switch: the grouped kernel runs its
    arithmetic) and against the oracle."""
    xs = [to_dev_bf16(x) for x in xs_bits]
    q = [fq.quantize_weight_channelwise(to_dev_bf16(w)) for w in ws_bits]
    ys = fq.quant_linear_group_m1(xs, [a for a, _ in q], [b for _, b in q])
    monkeypatch.setenv("FP8W8A8_GEMV_M1", "1")
    sep = [fq.quant_linear(x, a, b) for x, (a, b) in zip(xs, q)]
    monkeypatch.delenv("FP8W8A8_GEMV_M1")
    torch.cuda.synchronize()
    for i, (x, (a, b)) in enumerate(zip(xs_bits, q)):
        check_bytes(host_bits(ys[i]), host_bits(sep[i]), f"{what} item {i} vs alone")
        y64, _, _ = oracle.quant_linear_ref(x, host_bits(a), host_bits(b))
        check_close(host_bits(ys[i]), y64, f"{what} item {i} vs oracle")


def test_group_decode_layer(monkeypatch):
    """The decode layer's 7 Linears: also bit-identical to the default
    separate calls (for these shapes the default kernels give every wave
    whole rows and so the same summation order)."""
    xs, ws = zip(*(c2_inputs(1, j) for j in range(len(LAYER_SHAPES))))
    _check_group(xs, ws, "decode layer", monkeypatch)
    xd = [to_dev_bf16(x) for x in xs]
    q = [fq.quantize_weight_channelwise(to_dev_bf16(w)) for w in ws]
    ys = fq.quant_linear_group_m1(xd, [a for a, _ in q], [b for _, b in q])
    sep = [fq.quant_linear(x, a, b) for x, (a, b) in zip(xd, q)]
    torch.cuda.synchronize()
    for i in range(len(ys)):
        check_bytes(host_bits(ys[i]), host_bits(sep[i]), f"decode layer item {i} vs default")


@pytest.mark.parametrize("grid,order", [(None, "0"), ("7", "1"), ("1024", "0"),
                                        ("1024", "1")])
@pytest.mark.parametrize("seed", [0, 1])
def test_group_ragged_shapes(seed, grid, order, monkeypatch):
    """Also on a persistent grid (7 workgroups each looping over hundreds of
    work units, whose LDS staging is reused unit after unit; 1024) and with
    the items reordered longest-row first."""
    if grid is not None:
        monkeypatch.setenv("FP8W8A8_GROUP_GRID", grid)
    monkeypatch.setenv("FP8W8A8_GROUP_SORT", order)
    rng = np.random.default_rng(300 + seed)
    shapes = [(16, 128), (48, 4224), (1040, 2176), (4112, 6272), (2064, 12288),
              (272, 384), (16, 12288), (6144, 4096), (32, 8192)]
    xs, ws = [], []
    for n, k in shapes:
        scale = 10.0 ** rng.uniform(-3, 3)
        xs.append(bf16_from_f64(rng.standard_normal((1, k)) * scale *
                                np.where(rng.random((1, k)) < 0.01, 20.0, 1.0)))
        ws.append(bf16_from_f64(rng.standard_normal((n, k)) * 0.02))
    order = rng.permutation(len(shapes))
    _check_group([xs[i] for i in order], [ws[i] for i in order], f"ragged seed {seed}",
                 monkeypatch)


def test_group_zero_row_and_single_item(monkeypatch):
    x = np.zeros((1, 4096), np.uint16)
    w = bf16_from_f64(np.random.default_rng(5).standard_normal((64, 4096)) * 0.02)
    _check_group([x], [w], "zero row", monkeypatch)
    xs = [bf16_from_f64(np.random.default_rng(6 + i).standard_normal((1, 12288)))
          for i in range(16)]
    ws = [bf16_from_f64(np.random.default_rng(40 + i).standard_normal((16, 12288)) * 0.02)
          for i in range(16)]
    _check_group(xs, ws, "16 items", monkeypatch)
