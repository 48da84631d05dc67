"""GPU parity of the FP8 E4M3 KV-cache codec against the oracle, through the
C ABI (Python binding).  Codes, scales and the read-back bf16 values are
exact decisions on both sides (the same encoder definition; one float32
product and one bf16 rounding), so every comparison is bit-exact."""

import ctypes

import numpy as np
import pytest
import torch

import fp8_w8a8_dynamic_amd as fq
from oracle import DECODE_TABLE, check_bytes
from oracle.kvcache import kv_fp8_dequant_ref, kv_fp8_quant_ref
from tests.gpu_util import host_bits, to_dev_bf16, to_dev_f32, to_dev_u8
from workloads import bf16_from_f64, kv_inputs

pytestmark = pytest.mark.gpu

GROUPS = [8, 16, 32, 64, 128, 256, 512]


def _roundtrip(x_bits, group, ldx=None):
    x = to_dev_bf16(x_bits)
    if ldx is not None:
        wide = torch.zeros((x_bits.shape[0], ldx), dtype=torch.bfloat16, device="cuda")
        wide[:, : x_bits.shape[1]] = x
        x = wide[:, : x_bits.shape[1]]
    codes, scales = fq.kv_quantize_fp8(x, group)
    back = fq.kv_dequantize_fp8(codes, scales, group)
    torch.cuda.synchronize()
    return host_bits(codes), host_bits(scales), host_bits(back)


def _check(x_bits, group, codes, scales, back, what):
    rc, rs = kv_fp8_quant_ref(x_bits, group)
    check_bytes(scales.view(np.uint32), rs.view(np.uint32), what + " scales")
    check_bytes(codes, rc, what + " codes")
    check_bytes(back, kv_fp8_dequant_ref(rc, rs, group), what + " read back")


def test_cache_window_full_size():
    """A 32768-token K cache window (8 KV heads x 128), one scale per head:
    the size the benchmark reads back."""
    x = kv_inputs(32768, 1024, seed=0)
    c, s, b = _roundtrip(x, 128)
    _check(x, 128, c, s, b, "32768x1024 g128")


@pytest.mark.parametrize("group", GROUPS)
@pytest.mark.parametrize("t,w", [(1, 1024), (5, 512), (7, 1536), (3, 4096), (9, 2048)])
def test_groups_and_widths(t, w, group):
    if w % group:
        pytest.skip("group does not divide the width")
    x = kv_inputs(t, w, seed=t * 31 + w + group)
    c, s, b = _roundtrip(x, group)
    _check(x, group, c, s, b, f"{t}x{w} g{group}")


@pytest.mark.parametrize("w,group", [(8, 8), (520, 8), (1000, 8), (1040, 16), (2600, 8),
                                     (576, 64), (1664, 128)])
def test_ragged_last_chunk_and_strided_rows(w, group):
    x = kv_inputs(6, w, seed=w)
    c, s, b = _roundtrip(x, group, ldx=w + 24)
    _check(x, group, c, s, b, f"ragged {w} g{group}")


def test_groups_on_different_divisor_paths_in_one_wave():
    """Adjacent groups with scales inside and outside the quantizer's fast
    range (and all-zero, -0 and subnormal groups) in the same row."""
    rng = np.random.default_rng(7)
    w, group = 1024, 64
    x = rng.standard_normal((4, w))
    mags = [1.0, 1e25, 1e-25, 0.0, 3e38, 2.0 ** -120, 448.0, 1e-3,
            1.0, 0.0, 1e20, 1e-20, 7.0, 2.0 ** 100, 2.0 ** -100, 1.0]
    for j, m in enumerate(mags):
        x[:, j * group:(j + 1) * group] *= m * 0.25
    xb = bf16_from_f64(x)
    xb[1, 3 * group:4 * group] = 0x8000                    # a -0 group
    xb[2, 9 * group:10 * group:2] = 0x8001                 # tiny negatives
    c, s, b = _roundtrip(xb, group)
    _check(xb, group, c, s, b, "mixed groups")


def test_every_code_reads_back_exactly():
    codes = np.array([[c for c in range(256) if c not in (0x7F, 0xFF)] * 4], np.uint8)
    codes = codes.reshape(8, 127)[:, :120].copy()          # 8 rows x 120 codes
    rng = np.random.default_rng(8)
    scales = (rng.uniform(0.5, 2, (8, 15)) * 2.0 ** rng.integers(-60, 60, (8, 15)))
    scales = scales.astype(np.float32)
    scales[0, 0] = 0.0
    scales[1, :] = 2.0 ** -133                             # subnormal products
    got = fq.kv_dequantize_fp8(to_dev_u8(codes), to_dev_f32(scales), 8)
    torch.cuda.synchronize()
    check_bytes(host_bits(got), kv_fp8_dequant_ref(codes, scales, 8), "every code")


def test_append_into_a_cache_tail():
    """Quantizing new tokens straight into the tail of an existing cache
    leaves the earlier entries untouched."""
    w, group, t0, t1 = 1024, 128, 100, 37
    x = kv_inputs(t0 + t1, w, seed=5)
    cache = torch.full((256, w), 0x11, dtype=torch.uint8, device="cuda")
    cscale = torch.full((256, w // group), -1.0, dtype=torch.float32, device="cuda")
    fq.kv_quantize_fp8(to_dev_bf16(x[:t0]), group, cache[:t0], cscale[:t0])
    fq.kv_quantize_fp8(to_dev_bf16(x[t0:]), group, cache[t0:t0 + t1], cscale[t0:t0 + t1])
    torch.cuda.synchronize()
    rc, rs = kv_fp8_quant_ref(x, group)
    check_bytes(host_bits(cache[:t0 + t1]), rc, "cache codes")
    check_bytes(host_bits(cscale[:t0 + t1]).view(np.uint32), rs.view(np.uint32), "cache scales")
    assert torch.all(cache[t0 + t1:] == 0x11) and torch.all(cscale[t0 + t1:] == -1.0)


def test_binding_and_abi_reject_bad_arguments():
    x = to_dev_bf16(kv_inputs(4, 1024, seed=1))
    with pytest.raises(ValueError):
        fq.kv_quantize_fp8(x, 96)
    lib = fq.load_library()
    s = torch.empty((4, 8), dtype=torch.float32, device="cuda")
    st = lib.fp8w8a8_kv_quantize_fp8(x.data_ptr(), 4, 1024, 1024, 128, x.data_ptr(),
                                     s.data_ptr(), None)
    assert st == 4                                         # codes over kv: ERR_ALIAS
    st = lib.fp8w8a8_kv_quantize_fp8(x.data_ptr(), 4, 1024, 1024, 1024, x.data_ptr() + 8192 * 2,
                                     s.data_ptr(), None)
    assert st == 2                                         # group above 512: ERR_SHAPE


# ---- INT8 group-wise cache with a BF16 residual window ----------------------

from oracle.kvcache import kv_int8_dequant_ref, kv_int8_quant_ref, kv_int8_read_ref


def _int8(x_bits, group, ldx=None):
    x = to_dev_bf16(x_bits)
    if ldx is not None:
        wide = torch.zeros((x_bits.shape[0], ldx), dtype=torch.bfloat16, device="cuda")
        wide[:, : x_bits.shape[1]] = x
        x = wide[:, : x_bits.shape[1]]
    q, s, m = fq.kv_quantize_int8(x, group)
    torch.cuda.synchronize()
    return q, s, m


def _check_int8(x_bits, group, q, s, m, what):
    rq, rs, rm = kv_int8_quant_ref(x_bits, group)
    check_bytes(host_bits(s).view(np.uint32), rs.view(np.uint32), what + " scales")
    check_bytes(host_bits(m).view(np.uint32), rm.view(np.uint32), what + " mins")
    check_bytes(host_bits(q), rq, what + " codes")
    back = fq.kv_read_int8(q, s, m, group=group)
    torch.cuda.synchronize()
    check_bytes(host_bits(back), kv_int8_dequant_ref(rq, rs, rm, group), what + " read")


def test_int8_cache_window_full_size():
    """A 32768-token window as the cache holds it: 32640 tokens of INT8
    history (groups of 64) and the newest 128 as the bf16 tail."""
    x = kv_inputs(32768, 1024, seed=2)
    hist, tail = x[:-128], x[-128:]
    q, s, m = _int8(hist, 64)
    _check_int8(hist, 64, q, s, m, "int8 history")
    out = fq.kv_read_int8(q, s, m, tail=to_dev_bf16(tail), group=64)
    torch.cuda.synchronize()
    rq, rs, rm = kv_int8_quant_ref(hist, 64)
    check_bytes(host_bits(out), kv_int8_read_ref(rq, rs, rm, tail, 64), "int8 read")


@pytest.mark.parametrize("group", GROUPS)
@pytest.mark.parametrize("t,w", [(1, 1024), (5, 512), (7, 1536), (9, 2048)])
def test_int8_groups_and_widths(t, w, group):
    if w % group:
        pytest.skip("group does not divide the width")
    x = kv_inputs(t, w, seed=t * 17 + w + group)
    q, s, m = _int8(x, group)
    _check_int8(x, group, q, s, m, f"int8 {t}x{w} g{group}")


@pytest.mark.parametrize("w,group", [(8, 8), (520, 8), (1040, 16), (576, 64)])
def test_int8_ragged_and_strided(w, group):
    x = kv_inputs(5, w, seed=w + 3)
    q, s, m = _int8(x, group, ldx=w + 40)
    _check_int8(x, group, q, s, m, f"int8 ragged {w}")


def test_int8_extreme_and_constant_groups():
    rng = np.random.default_rng(21)
    w, group = 1024, 64
    x = rng.standard_normal((3, w))
    mags = [1.0, 1e30, 1e-30, 0.0, 1e37, 2.0 ** -125, 448.0, 1e-3,
            1.0, 1e20, 1e-20, 7.0, 2.0 ** 100, 2.0 ** -100, 5.0, 0.5]
    for j, mg in enumerate(mags):
        x[:, j * group:(j + 1) * group] *= mg
    xb = bf16_from_f64(x)
    xb[0, 0:64] = 0x3F80                                    # constant +1
    xb[1, 64:128] = 0x8000                                  # all -0
    xb[2, 128:192:3] = 0x8001                               # tiny negatives in a tiny group
    q, s, m = _int8(xb, group)
    _check_int8(xb, group, q, s, m, "int8 extremes")


def test_int8_every_byte_reads_back_exactly():
    codes = np.tile(np.arange(256, dtype=np.uint8), (6, 2))   # 6 x 512
    rng = np.random.default_rng(22)
    scales = (rng.uniform(0.5, 2, (6, 8)) * 2.0 ** rng.integers(-60, 60, (6, 8))).astype(np.float32)
    mins = (-rng.uniform(0, 300, (6, 8)) * scales).astype(np.float32)
    scales[0, 0] = 0.0
    mins[1, :] = -0.0
    got = fq.kv_read_int8(to_dev_u8(codes), to_dev_f32(scales), to_dev_f32(mins), group=64)
    torch.cuda.synchronize()
    check_bytes(host_bits(got), kv_int8_dequant_ref(codes, scales, mins, 64), "every byte")


def test_int8_store_append_then_read_with_tail():
    """History built in two appends into a preallocated store, then read
    with a strided tail; rows beyond the store's fill stay untouched."""
    w, group = 1024, 64
    x = kv_inputs(300, w, seed=9)
    codes = torch.full((512, w), 7, dtype=torch.uint8, device="cuda")
    sc = torch.full((512, w // group), -2.0, dtype=torch.float32, device="cuda")
    mn = torch.full((512, w // group), -3.0, dtype=torch.float32, device="cuda")
    fq.kv_quantize_int8(to_dev_bf16(x[:150]), group, codes[:150], sc[:150], mn[:150])
    fq.kv_quantize_int8(to_dev_bf16(x[150:200]), group, codes[150:200], sc[150:200],
                        mn[150:200])
    tail_wide = torch.zeros((100, w + 64), dtype=torch.bfloat16, device="cuda")
    tail_wide[:, :w] = to_dev_bf16(x[200:])
    out = fq.kv_read_int8(codes[:200], sc[:200], mn[:200], tail=tail_wide[:, :w], group=group)
    torch.cuda.synchronize()
    rq, rs, rm = kv_int8_quant_ref(x[:200], group)
    check_bytes(host_bits(out), kv_int8_read_ref(rq, rs, rm, x[200:], group), "append+read")
    assert torch.all(codes[200:] == 7) and torch.all(sc[200:] == -2.0)
