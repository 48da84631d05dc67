"""GPU parity of the single-call RMSNorm -> Linear and SiLU-gate -> Linear
entries (rmsnorm_quant_linear, swiglu_quant_linear) through the C ABI.

At decode sizes the norm or the activation runs inside the GEMV's
activation staging; elsewhere the call runs the stand-alone pre-step kernel
into the workspace and then the Linear.  Either way the result is defined
as the two-step composition fp8_linear(*rmsnorm_quantize(...)) (or
swiglu_quantize), so the bar is bit-identity with it, on every element.
The two-step path's own parity with the oracle is covered by the norm,
activation and Linear tests; here the fused result is also held within the
Linear's 1e-2 bound of the oracle's whole chain.
"""

import numpy as np
import pytest
import torch

import fp8_w8a8_dynamic_amd as fq
import oracle
from oracle import check_close
from oracle.norm import rmsnorm_quant_ref
from oracle.swiglu import swiglu_quant_ref
from tests.gpu_util import host_bits, to_dev_bf16
from workloads import bf16_from_f64, norm_inputs, swiglu_inputs, weight_bf16

pytestmark = pytest.mark.gpu

EPS = 1e-6


def _weights(n, k, seed):
    w = weight_bf16(9, seed, 0, n, k)
    qw, sw = fq.quantize_weight_channelwise(to_dev_bf16(w))
    return qw, sw


def _norm_pair(x_bits, g_bits, qw, sw, eps=EPS):
    x, g = to_dev_bf16(x_bits), to_dev_bf16(g_bits)
    fused = fq.rmsnorm_quant_linear(x, g, eps, qw, sw)
    qx, sx = fq.rmsnorm_quantize(x, g, eps)
    two = fq.fp8_linear(qx, sx, qw, sw)
    torch.cuda.synchronize()
    return host_bits(fused), host_bits(two)


def _swiglu_pair(g_bits, u_bits, qw, sw):
    g, u = to_dev_bf16(g_bits), to_dev_bf16(u_bits)
    fused = fq.swiglu_quant_linear(g, u, qw, sw)
    qh, sh = fq.swiglu_quantize(g, u)
    two = fq.fp8_linear(qh, sh, qw, sw)
    torch.cuda.synchronize()
    return host_bits(fused), host_bits(two)


def _same(a, b, what):
    bad = np.flatnonzero(a.ravel() != b.ravel())
    assert bad.size == 0, (f"{what}: {bad.size} of {a.size} outputs differ from the "
                           f"two-step path, first at {np.unravel_index(bad[0], a.shape)}")


# -- RMSNorm -> Linear ---------------------------------------------------------

@pytest.mark.parametrize("m,n,k", [(1, 4096, 4096), (2, 1024, 4096), (3, 512, 4096),
                                   (4, 4096, 4096), (1, 256, 512), (2, 384, 1536),
                                   (1, 1024, 16384), (1, 512, 4224), (5, 1024, 4096),
                                   (17, 512, 1024), (64, 1024, 4096)])
def test_norm_linear_matches_two_step(m, n, k):
    x, g = norm_inputs(m, k, seed=m + k)
    qw, sw = _weights(n, k, 1)
    fused, two = _norm_pair(x, g, qw, sw)
    _same(fused, two, f"norm m={m} n={n} k={k}")


@pytest.mark.parametrize("m", [5, 8, 16])
def test_norm_linear_every_fused_row_count(m, monkeypatch):
    # Up to 16 rows the GEMV can take the norm; by default it serves m <= 4.
    monkeypatch.setenv("FP8W8A8_FORCE_PATH", "gemv")
    x, g = norm_inputs(m, 1024, seed=m)
    qw, sw = _weights(512, 1024, 2)
    fused, two = _norm_pair(x, g, qw, sw)
    _same(fused, two, f"forced gemv m={m}")


def test_norm_linear_extreme_rows():
    # Rows whose float32 sum of squares leaves the trusted range take the
    # exactly scaled path inside the fused staging; a zero row with eps = 0
    # gives t = 0 and a zero scale.
    k, n = 2048, 512
    x, g = norm_inputs(4, k, seed=5)
    xv = oracle.bf16_bits_to_f32(x).astype(np.float64)
    xv[0] *= 2.0 ** 100
    xv[1] *= 2.0 ** -100
    xv[2] = 0.0
    xv[3, ::7] = 3.0e38
    xb = bf16_from_f64(xv)
    qw, sw = _weights(n, k, 3)
    for eps in (EPS, 0.0):
        for rows in ([0], [1], [2], [3], [0, 1, 2, 3]):
            fused, two = _norm_pair(np.ascontiguousarray(xb[rows]), g, qw, sw, eps)
            _same(fused, two, f"extreme rows {rows} eps={eps}")


def test_norm_linear_vs_oracle_chain():
    m, n, k = 2, 1024, 4096
    x, g = norm_inputs(m, k, seed=11)
    w = weight_bf16(9, 4, 1, n, k)
    qw, sw = fq.quantize_weight_channelwise(to_dev_bf16(w))
    y = fq.rmsnorm_quant_linear(to_dev_bf16(x), to_dev_bf16(g), EPS, qw, sw)
    qx, sx, _ = rmsnorm_quant_ref(x, g, EPS)
    rqw, rsw = oracle.quant_weight_ref(w)
    ref = oracle.linear_ref(qx, sx, rqw, rsw)
    check_close(host_bits(y), ref, "rmsnorm_quant_linear vs oracle")


def test_norm_linear_strided_input_and_output():
    m, n, k = 3, 512, 2048
    x, g = norm_inputs(m, k, seed=12)
    qw, sw = _weights(n, k, 5)
    wide = torch.zeros((m, k + 256), dtype=torch.bfloat16, device="cuda")
    wide[:, :k] = to_dev_bf16(x)
    yw = torch.full((m, n + 64), 7.0, dtype=torch.bfloat16, device="cuda")
    fq.rmsnorm_quant_linear(wide[:, :k], to_dev_bf16(g), EPS, qw, sw, out=yw[:, :n])
    fused, two = _norm_pair(x, g, qw, sw)
    got = host_bits(yw)
    _same(got[:, :n], two, "strided")
    assert (got[:, n:] == host_bits(torch.tensor(7.0, dtype=torch.bfloat16))).all()


# -- SiLU-gate -> Linear -------------------------------------------------------

@pytest.mark.parametrize("m,n,k", [(1, 4096, 12288), (2, 1024, 8192), (4, 512, 4096),
                                   (3, 256, 1152), (1, 512, 128), (2, 4096, 12288),
                                   (9, 512, 1024), (64, 1024, 12288)])
def test_swiglu_linear_matches_two_step(m, n, k):
    gb, ub = swiglu_inputs(m, k, seed=m + k)
    qw, sw = _weights(n, k, 6)
    fused, two = _swiglu_pair(gb, ub, qw, sw)
    _same(fused, two, f"swiglu m={m} n={n} k={k}")


@pytest.mark.parametrize("m", [5, 16])
def test_swiglu_linear_every_fused_row_count(m, monkeypatch):
    monkeypatch.setenv("FP8W8A8_FORCE_PATH", "gemv")
    gb, ub = swiglu_inputs(m, 1024, seed=m)
    qw, sw = _weights(512, 1024, 7)
    fused, two = _swiglu_pair(gb, ub, qw, sw)
    _same(fused, two, f"forced gemv m={m}")


def test_swiglu_linear_deep_gates():
    # Gates far below -44 take the exponent-shifted form of silu.
    m, k, n = 2, 4096, 512
    gb, ub = swiglu_inputs(m, k, seed=3)
    gv = oracle.bf16_bits_to_f32(gb).astype(np.float64)
    gv[0, ::5] = -60.0 - np.arange(gv[0, ::5].size) % 40
    gv[1, 100:200] = -100.0
    fused, two = _swiglu_pair(bf16_from_f64(gv), ub, *_weights(n, k, 8))
    _same(fused, two, "deep gates")


def test_swiglu_linear_vs_oracle_chain():
    m, n, k = 1, 1024, 12288
    gb, ub = swiglu_inputs(m, k, seed=21)
    w = weight_bf16(9, 9, 1, n, k)
    qw, sw = fq.quantize_weight_channelwise(to_dev_bf16(w))
    y = fq.swiglu_quant_linear(to_dev_bf16(gb), to_dev_bf16(ub), qw, sw)
    qh, sh, _ = swiglu_quant_ref(gb, ub)
    rqw, rsw = oracle.quant_weight_ref(w)
    ref = oracle.linear_ref(qh, sh, rqw, rsw)
    check_close(host_bits(y), ref, "swiglu_quant_linear vs oracle")


def test_swiglu_linear_packed_halves():
    # gate and up as the two halves of one gate_up output row.
    m, k, n = 2, 4096, 512
    gb, ub = swiglu_inputs(m, k, seed=4)
    gu = torch.cat([to_dev_bf16(gb), to_dev_bf16(ub)], dim=1)
    qw, sw = _weights(n, k, 10)
    y = fq.swiglu_quant_linear(gu[:, :k], gu[:, k:], qw, sw)
    fused, two = _swiglu_pair(gb, ub, qw, sw)
    _same(host_bits(y), two, "packed halves")


def test_empty_and_workspace_reuse():
    qw, sw = _weights(512, 1024, 11)
    x = torch.zeros((0, 1024), dtype=torch.bfloat16, device="cuda")
    g = torch.ones(1024, dtype=torch.bfloat16, device="cuda")
    assert fq.rmsnorm_quant_linear(x, g, EPS, qw, sw).shape == (0, 512)
    assert fq.swiglu_quant_linear(x, x, qw, sw).shape == (0, 512)
    ws = torch.empty(fq.workspace_bytes(64, 512, 1024, 2), dtype=torch.uint8, device="cuda")
    for m in (64, 1, 40):
        xb, gb = norm_inputs(m, 1024, seed=m)
        y = fq.rmsnorm_quant_linear(to_dev_bf16(xb), to_dev_bf16(gb), EPS, qw, sw,
                                    workspace=ws)
        _, two = _norm_pair(xb, gb, qw, sw)
        _same(host_bits(y), two, f"workspace reuse m={m}")
