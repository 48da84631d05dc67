"""GPU parity of the fused SiLU-gated activation -> per-token quantization
kernel against the oracle (calls through the C ABI via the Python binding).

The bar, derived from the arithmetic: the kernel evaluates silu in float32
with a relative error below 2^-16 (the rounding of g log2(e), scaled by |g|
up to the range where the result is still a normal float, plus a few ulps
of exp2, rcp and the products), the oracle in float64; both round s =
silu(g) and then h = s * u to bfloat16.  So s may round the other way than
the oracle's only where the oracle's silu lies within 2^-16 (relative) of a
bfloat16 rounding midpoint, and each such h must then equal the oracle's h
computed from that other rounding of s; everything else is bit-identical.
Codes and scales are bit-identical to the oracle's quantizer applied to the
kernel's own h, and to the oracle's outright on every row whose h matches.
"""

import ctypes

import numpy as np
import pytest
import torch

import fp8_w8a8_dynamic_amd as fq
import oracle
from oracle import bf16_bits_to_f32, check_bytes, f64_to_bf16_bits
from oracle.swiglu import swiglu_ref
from tests.gpu_util import host_bits, to_dev_bf16
from workloads import bf16_from_f64, swiglu_inputs, weight_bf16

pytestmark = pytest.mark.gpu

BAND = 2.0 ** -16


def _gpu(g_bits, u_bits, with_h=True, packed=False):
    m, n = g_bits.shape
    if packed:
        gu = to_dev_bf16(np.concatenate([g_bits, u_bits], axis=1))
        g, u = gu[:, :n], gu[:, n:]
        assert g.stride(0) == 2 * n and u.stride(0) == 2 * n
    else:
        g, u = to_dev_bf16(g_bits), to_dev_bf16(u_bits)
    if with_h:
        qh, sh, h = fq.swiglu_quantize(g, u, return_h=True)
    else:
        qh, sh = fq.swiglu_quantize(g, u)
        h = None
    torch.cuda.synchronize()
    return host_bits(qh), host_bits(sh), (host_bits(h) if h is not None else None)


def check_swiglu(g_bits, u_bits, qh, sh, h, what):
    h_or, s_or, a = swiglu_ref(g_bits, u_bits)
    mism = h != h_or
    n_mis = int(mism.sum())
    if n_mis:
        rows, cols = np.nonzero(mism)
        a_m, s_m = a[mism], s_or[mism]
        sb = bf16_bits_to_f32(s_m).astype(np.float64)
        away = np.abs(a_m) > np.abs(sb)
        nb = np.where(away, s_m.astype(np.int32) + 1, s_m.astype(np.int32) - 1)
        nb = nb.astype(np.uint16)
        mid = (sb + bf16_bits_to_f32(nb).astype(np.float64)) / 2
        near = (np.abs(a_m - mid) <= BAND * np.abs(a_m)) & (a_m != sb)
        u = bf16_bits_to_f32(u_bits[mism]).astype(np.float64)
        h_alt = f64_to_bf16_bits(bf16_bits_to_f32(nb).astype(np.float64) * u)
        bad = ~((h[mism] == h_alt) & near)
        assert not bad.any(), (
            f"{what}: {int(bad.sum())} of {n_mis} differing outputs are not the other "
            f"rounding of silu near a midpoint; first at row {rows[bad][0]}, col "
            f"{cols[bad][0]}: g {bf16_bits_to_f32(g_bits[mism][bad][:1])[0]!r} gpu "
            f"{h[mism][bad][0]:#06x} oracle {h_or[mism][bad][0]:#06x}")
        assert n_mis <= max(8, h.size // 1000), f"{what}: {n_mis} mismatches"
    rq, rs = oracle.quant_act_ref(h)
    check_bytes(sh.view(np.uint32), rs.view(np.uint32), what + " scales (own h)")
    check_bytes(qh, rq, what + " codes (own h)")
    oq, os_ = oracle.quant_act_ref(h_or)
    ok_rows = ~mism.any(axis=1)
    check_bytes(qh[ok_rows], oq[ok_rows], what + " codes (oracle)")
    check_bytes(sh[ok_rows].view(np.uint32), os_[ok_rows].view(np.uint32),
                what + " scales (oracle)")
    assert np.all(np.abs(sh.astype(np.float64) - os_) <= 2.0 ** -6 * os_)
    return n_mis


def test_prefill_chunk_full_size():
    """down_proj's input for a 4096-token prefill chunk: the halves of the
    packed gate_up output [4096, 24576], in the launch configuration the
    benchmark times."""
    g, u = swiglu_inputs(4096, 12288, seed=0)
    qh, sh, h = _gpu(g, u, packed=True)
    n = check_swiglu(g, u, qh, sh, h, "prefill 4096x12288")
    print(f"h mismatches near rounding midpoints: {n} of {h.size}")


SHAPES = [(1, 8), (3, 1024), (5, 2048), (7, 4096), (9, 8192), (6, 12288),
          (5, 12296), (3, 16384), (2, 16392), (4, 1000), (17, 520), (1, 12288)]


@pytest.mark.parametrize("m,n", SHAPES)
def test_shapes_and_kernel_variants(m, n):
    """Every (vectors per lane, waves per row) variant, ragged tails, rows
    that leave waves of a workgroup idle, and the two-pass kernel."""
    g, u = swiglu_inputs(m, n, seed=m * 7 + n)
    qh, sh, h = _gpu(g, u)
    check_swiglu(g, u, qh, sh, h, f"{m}x{n}")


@pytest.mark.parametrize("n", [4096, 12288, 16392])
def test_deep_negative_gates(n):
    """Gates below -44 (the other silu form), mixed into slices with common
    values, down to where silu underflows bf16; and rows made only of them."""
    rng = np.random.default_rng(n)
    g = rng.standard_normal((6, n)) * 1.5
    mask = rng.random((6, n)) < 0.05
    g[mask] = rng.uniform(-120.0, -40.0, mask.sum())
    g[3] = rng.uniform(-110.0, -44.5, n)
    g[4] = np.linspace(-200.0, 200.0, n)
    gb = bf16_from_f64(g)
    ub = bf16_from_f64(rng.standard_normal((6, n)) * 1.5)
    qh, sh, h = _gpu(gb, ub)
    check_swiglu(gb, ub, qh, sh, h, f"deep gates n={n}")


def test_extremes_zeros_and_signs():
    n = 256
    vals = np.array([0.0, -0.0, 3.0e38, -3.0e38, 1e-38, -1e-38, 88.0, -88.0,
                     44.0, -44.0, -43.75, -44.25, 1e-30, -1e-30, 7.0, -7.0])
    g = np.tile(vals, (4, n // vals.size))
    gb = bf16_from_f64(g)
    gb[:, 1::16] = 0x8000                                     # exact -0
    ub = bf16_from_f64(np.tile([1.0, -1.0, 2.5e-30, -3.0, 1e20, 0.0, -0.5, 8.0],
                               (4, n // 8)))
    ub[1] = 0                                                 # all-zero h row
    qh, sh, h = _gpu(gb, ub)
    check_swiglu(gb, ub, qh, sh, h, "extremes")
    assert sh[1] == 0


def test_without_h_and_packed_vs_separate():
    g, u = swiglu_inputs(40, 12288, seed=3)
    q1, s1, h1 = _gpu(g, u)
    q2, s2, _ = _gpu(g, u, with_h=False)
    q3, s3, h3 = _gpu(g, u, packed=True)
    assert np.array_equal(q1, q2) and np.array_equal(q1, q3) and np.array_equal(h1, h3)
    assert np.array_equal(s1.view(np.uint32), s2.view(np.uint32))
    assert np.array_equal(s1.view(np.uint32), s3.view(np.uint32))


def test_swiglu_then_down_linear():
    """The activation's codes and scales feed down_proj directly."""
    m, n, k_out = 48, 12288, 4096
    g, u = swiglu_inputs(m, n, seed=4)
    w = weight_bf16(7, 0, 6, k_out, n)
    qw, sw = fq.quantize_weight_channelwise(to_dev_bf16(w))
    qh, sh = fq.swiglu_quantize(to_dev_bf16(g), to_dev_bf16(u))
    y = fq.fp8_linear(qh, sh, qw, sw)
    torch.cuda.synchronize()
    ref = oracle.linear_ref(host_bits(qh), host_bits(sh), host_bits(qw), host_bits(sw))
    oracle.check_close(host_bits(y), ref, "swiglu -> down linear")


def test_binding_and_abi_reject_bad_arguments():
    g, u = swiglu_inputs(4, 64, seed=1)
    gd, ud = to_dev_bf16(g), to_dev_bf16(u)
    with pytest.raises(ValueError):
        fq.swiglu_quantize(gd, ud[:, :32])
    with pytest.raises(TypeError):
        fq.swiglu_quantize(gd.float(), ud)
    lib = fq.load_library()
    sh = torch.empty(4, dtype=torch.float32, device="cuda")
    st = lib.fp8w8a8_swiglu_quantize(gd.data_ptr(), 64, ud.data_ptr(), 64, 4, 64,
                                     gd.data_ptr(), sh.data_ptr(), None, 0, None)
    assert st == 4                                   # codes over gate: ERR_ALIAS
