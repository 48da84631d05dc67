"""GPU parity of the fused BF16 RMSNorm -> per-token quantization kernel
against the oracle (calls through the C ABI via the Python binding).

The bar, derived from the arithmetic: the kernel evaluates the
normalization in float32 (relative error below 2^-17 of t for rows up to a
few thousand elements), the oracle in float64, and both round t and then
gamma * t to bfloat16.  So t may round the other way than the oracle's only
where the oracle's t lies within 2^-17 (relative) of a bfloat16 rounding
midpoint, and each bf16 norm output y must then equal the oracle's y
computed from that other rounding of t (one or two bf16 steps away, as
gamma scales the step); everything else is bit-identical.  The quantization is an integer decision made on y: codes and
scales must be bit-identical to the oracle's quantizer applied to the
kernel's own y (the same precision on both sides), and to the oracle's codes
outright on every row whose y matches.
"""

import ctypes

import numpy as np
import pytest
import torch

import fp8_w8a8_dynamic_amd as fq
import oracle
from oracle import bf16_bits_to_f32, check_bytes, f64_to_bf16_bits
from oracle.norm import rmsnorm_ref
from tests.gpu_util import host_bits, to_dev_bf16, to_dev_f32, to_dev_u8
from workloads import LAYER_SHAPES, bf16_from_f64, norm_inputs, weight_bf16

pytestmark = pytest.mark.gpu

BAND = 2.0 ** -17


def _gpu_norm(x_bits, g_bits, eps, normed=True, ldx=None):
    x = to_dev_bf16(x_bits)
    if ldx is not None and ldx != x_bits.shape[1]:
        wide = torch.zeros((x_bits.shape[0], ldx), dtype=torch.bfloat16, device="cuda")
        wide[:, : x_bits.shape[1]] = x
        x = wide[:, : x_bits.shape[1]]
        assert x.stride(0) == ldx
    g = to_dev_bf16(g_bits)
    if normed:
        qx, sx, y = fq.rmsnorm_quantize(x, g, eps, return_normed=True)
    else:
        qx, sx = fq.rmsnorm_quantize(x, g, eps)
        y = None
    torch.cuda.synchronize()
    return host_bits(qx), host_bits(sx), (host_bits(y) if y is not None else None)


def _other_rounding(t, t_bits):
    """The bfloat16 neighbour of t's nearest value (t_bits) on t's side, and
    whether t lies within BAND (relative) of the midpoint between the two."""
    tb = bf16_bits_to_f32(t_bits).astype(np.float64)
    away = np.abs(t) > np.abs(tb)                 # t beyond tb, away from 0
    nb = np.where(away, t_bits.astype(np.int32) + 1,
                  t_bits.astype(np.int32) - 1).astype(np.uint16)
    nbv = bf16_bits_to_f32(nb).astype(np.float64)
    mid = (tb + nbv) / 2
    near = (np.abs(t - mid) <= BAND * np.abs(t)) & (t != tb)
    return nb, near


def check_norm(x_bits, g_bits, eps, qx, sx, y, what):
    y_or, t_or = rmsnorm_ref(x_bits, g_bits, eps)
    mism = y != y_or
    n_mis = int(mism.sum())
    if n_mis:
        # Each differing y must be exactly the oracle's y with the other
        # rounding of t, at an element whose t is within float32 error of
        # that rounding's midpoint.
        rows, cols = np.nonzero(mism)
        t_m = t_or[mism]
        nb, near = _other_rounding(t_m, f64_to_bf16_bits(t_m))
        g = bf16_bits_to_f32(g_bits).astype(np.float64)[cols]
        y_alt = f64_to_bf16_bits(g * bf16_bits_to_f32(nb).astype(np.float64))
        bad = ~((y[mism] == y_alt) & near)
        assert not bad.any(), (
            f"{what}: {int(bad.sum())} of {n_mis} differing outputs are not the "
            f"other rounding of t near a midpoint; first at row {rows[bad][0]}, "
            f"col {cols[bad][0]}: gpu {y[mism][bad][0]:#06x} oracle "
            f"{y_or[mism][bad][0]:#06x} other {y_alt[bad][0]:#06x} t {t_m[bad][0]!r}")
        assert n_mis <= max(8, y.size // 1000), f"{what}: {n_mis} mismatches"
    # Quantization of the kernel's own y: bit-exact.
    rq, rs = oracle.quant_act_ref(y)
    check_bytes(sx.view(np.uint32), rs.view(np.uint32), what + " scales (own y)")
    check_bytes(qx, rq, what + " codes (own y)")
    # Against the oracle outright: exact on every row whose y matches; a row
    # with a differing y has its amax off by at most two bf16 steps.
    oq, os_ = oracle.quant_act_ref(y_or)
    ok_rows = ~mism.any(axis=1)
    check_bytes(qx[ok_rows], oq[ok_rows], what + " codes (oracle)")
    check_bytes(sx[ok_rows].view(np.uint32), os_[ok_rows].view(np.uint32),
                what + " scales (oracle)")
    rel = np.abs(sx.astype(np.float64) - os_) <= 2.0 ** -6 * os_
    assert np.all(rel), f"{what}: scale off by more than two bf16 steps"
    return n_mis


SPLITS = ["1", "2", "4"]


@pytest.mark.parametrize("split", [None] + SPLITS)
def test_prefill_chunk_full_size(split, monkeypatch):
    """The input norm of a 4096-token prefill chunk (hidden 4096): in the
    launch configuration the benchmark times (split None: the library's
    choice) and with each row split over 1, 2 or 4 waves."""
    if split is not None:
        monkeypatch.setenv("FP8W8A8_NORM_SPLIT", split)
    x, g = norm_inputs(4096, 4096, seed=0)
    qx, sx, y = _gpu_norm(x, g, 1e-6)
    n = check_norm(x, g, 1e-6, qx, sx, y, "prefill 4096x4096")
    print(f"y mismatches near rounding midpoints: {n} of {y.size}")


SHAPES = [(1, 4096), (3, 8), (5, 16), (7, 520), (64, 512), (5, 2048),
          (33, 4104), (2, 8192), (9, 12288), (6, 12296), (3, 16400)]


@pytest.mark.parametrize("split", SPLITS)
@pytest.mark.parametrize("m,k", SHAPES)
def test_shapes_and_kernel_variants(m, k, split, monkeypatch):
    """Every register-resident variant (up to 8, 16, 32, 64 and 96 elements
    per lane and wave, rows split over 1, 2 or 4 waves, idle waves in the
    last workgroup), ragged tails, and the multi-pass kernel for longer
    rows."""
    monkeypatch.setenv("FP8W8A8_NORM_SPLIT", split)
    x, g = norm_inputs(m, k, seed=m + k)
    qx, sx, y = _gpu_norm(x, g, 1e-6)
    check_norm(x, g, 1e-6, qx, sx, y, f"{m}x{k}")


@pytest.mark.parametrize("split", SPLITS)
@pytest.mark.parametrize("eps", [0.0, 1e-6, 1e-2, 1.0, 1e30])
def test_eps_values(eps, split, monkeypatch):
    monkeypatch.setenv("FP8W8A8_NORM_SPLIT", split)
    x, g = norm_inputs(16, 1024, seed=21)
    qx, sx, y = _gpu_norm(x, g, eps)
    check_norm(x, g, eps, qx, sx, y, f"eps {eps}")


@pytest.mark.parametrize("split", SPLITS)
@pytest.mark.parametrize("scale", [2.0 ** -120, 2.0 ** -70, 1e-20, 1e20, 2.0 ** 100,
                                   3e38])
@pytest.mark.parametrize("eps", [0.0, 1e-6])
def test_extreme_row_magnitudes(scale, eps, split, monkeypatch):
    """Rows whose float32 sum of squares would overflow or underflow without
    the power-of-two prescaling (and, with eps, rows that eps dominates),
    next to ordinary rows in the same workgroup."""
    monkeypatch.setenv("FP8W8A8_NORM_SPLIT", split)
    rng = np.random.default_rng(31)
    k = 768
    x = bf16_from_f64(rng.standard_normal((6, k)) * scale * 0.25)
    x[1] = bf16_from_f64(rng.standard_normal(k))              # an ordinary row
    x[4] = bf16_from_f64(rng.standard_normal(k) * 3.0)
    g = bf16_from_f64(1.0 + 0.25 * rng.standard_normal(k))
    qx, sx, y = _gpu_norm(x, g, eps)
    check_norm(x, g, eps, qx, sx, y, f"rows x{scale:g} eps {eps}")


@pytest.mark.parametrize("split", SPLITS)
def test_zero_rows_and_signed_zeros(split, monkeypatch):
    monkeypatch.setenv("FP8W8A8_NORM_SPLIT", split)
    k = 256
    g = bf16_from_f64(np.linspace(-2.0, 2.0, k))
    x = np.zeros((4, k), np.uint16)
    x[1, ::3] = 0x8000                       # -0.0 entries
    x[3] = bf16_from_f64(np.linspace(-1.0, 1.0, k))
    for eps in (0.0, 1e-6):
        qx, sx, y = _gpu_norm(x, g, eps)
        check_norm(x, g, eps, qx, sx, y, f"zero rows eps {eps}")
        assert np.all(sx[:3] == 0)


@pytest.mark.parametrize("split", SPLITS)
def test_subnormal_rows(split, monkeypatch):
    monkeypatch.setenv("FP8W8A8_NORM_SPLIT", split)
    k = 512
    rng = np.random.default_rng(41)
    x = rng.integers(0, 128, (6, k)).astype(np.uint16)       # bf16 subnormals
    x |= (rng.integers(0, 2, (6, k)).astype(np.uint16) << 15)
    g = bf16_from_f64(1.0 + rng.standard_normal(k) * 0.1)
    for eps in (0.0, 1e-30):
        qx, sx, y = _gpu_norm(x, g, eps)
        check_norm(x, g, eps, qx, sx, y, f"subnormal rows eps {eps}")


def test_without_normed_output_and_strided_input():
    """Skipping the y store and reading rows with a stride do not change a
    single byte of the codes or scales."""
    x, g = norm_inputs(48, 4096, seed=5)
    q1, s1, y1 = _gpu_norm(x, g, 1e-6)
    q2, s2, _ = _gpu_norm(x, g, 1e-6, normed=False)
    q3, s3, y3 = _gpu_norm(x, g, 1e-6, ldx=4096 + 64)
    assert np.array_equal(q1, q2) and np.array_equal(s1.view(np.uint32),
                                                      s2.view(np.uint32))
    assert np.array_equal(q1, q3) and np.array_equal(y1, y3)
    assert np.array_equal(s1.view(np.uint32), s3.view(np.uint32))


def test_strided_normed_output():
    x, g = norm_inputs(8, 1024, seed=6)
    xd, gd = to_dev_bf16(x), to_dev_bf16(g)
    wide = torch.full((8, 1024 + 32), 7.0, dtype=torch.bfloat16, device="cuda")
    out = wide[:, :1024]
    qx, sx, y = fq.rmsnorm_quantize(xd, gd, 1e-6, out=out)
    torch.cuda.synchronize()
    assert y.data_ptr() == out.data_ptr()
    check_norm(x, g, 1e-6, host_bits(qx), host_bits(sx), host_bits(y), "strided y")
    assert torch.all(wide[:, 1024:] == 7.0)          # padding untouched


def test_norm_then_packed_qkv_linear():
    """The norm's codes and scales feed the q|k|v Linear directly: the
    product matches the oracle's Linear on the same (kernel-made) codes."""
    m, k = 64, 4096
    x, g = norm_inputs(m, k, seed=9)
    n = sum(s[1] for s in LAYER_SHAPES[:3])
    w = weight_bf16(6, 0, 0, n, k)
    qw, sw = fq.quantize_weight_channelwise(to_dev_bf16(w))
    qx, sx = fq.rmsnorm_quantize(to_dev_bf16(x), to_dev_bf16(g), 1e-6)
    y = fq.fp8_linear(qx, sx, qw, sw)
    torch.cuda.synchronize()
    ref = oracle.linear_ref(host_bits(qx), host_bits(sx), host_bits(qw), host_bits(sw))
    oracle.check_close(host_bits(y), ref, "norm -> qkv linear")


def test_binding_and_abi_reject_bad_arguments():
    x, g = norm_inputs(4, 64, seed=1)
    xd, gd = to_dev_bf16(x), to_dev_bf16(g)
    with pytest.raises(ValueError):
        fq.rmsnorm_quantize(xd, gd[:32], 1e-6)
    with pytest.raises(TypeError):
        fq.rmsnorm_quantize(xd.float(), gd, 1e-6)
    for eps in (-1.0, float("nan")):
        with pytest.raises(fq.Fp8W8A8Error):
            fq.rmsnorm_quantize(xd, gd, eps)
    # Codes written over the input are refused before any kernel runs.
    lib = fq.load_library()
    sx = torch.empty(4, dtype=torch.float32, device="cuda")
    st = lib.fp8w8a8_rmsnorm_quantize(xd.data_ptr(), 4, 64, 64, gd.data_ptr(),
                                      ctypes.c_float(1e-6), xd.data_ptr(),
                                      sx.data_ptr(), None, 0, None)
    assert st == 4
