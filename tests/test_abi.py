"""The C ABI: the library loads, exports every declared symbol, and rejects
bad arguments on the host before touching a device (CPU only: no call here
reaches a kernel)."""

import ctypes
import os
import re

import pytest

from fp8_w8a8_dynamic_amd import SIGNATURES, load_library

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8w8a8.h")

OK, ENULL, ESHAPE, EALIGN, EALIAS, EWS, EDEV, EHIP = range(8)
A = 1 << 20          # fake, 16-byte aligned "device" addresses (never used)


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(fp8w8a8_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    # FP8W8A8_ABI_TEST_LIBRARY names another build of the same library (the
    # host-sanitized one, tests/test_abi_sanitized.py); default: the product.
    path = os.environ.get("FP8W8A8_ABI_TEST_LIBRARY")
    return load_library(path) if path else load_library()


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert len(names) == 24
    for name in names:
        assert hasattr(lib, name), name
    assert sorted(SIGNATURES) == names


def test_status_strings(lib):
    for code in range(8):
        assert lib.fp8w8a8_status_string(code).decode().startswith("FP8W8A8_")
    assert b"unknown" in lib.fp8w8a8_status_string(99)


def _q(lib, fn, src, rows, k, ld, q, s):
    return getattr(lib, fn)(src, rows, k, ld, q, s, None)


@pytest.mark.parametrize("fn", ["fp8w8a8_quantize_act_per_token",
                                "fp8w8a8_quantize_weight_channelwise"])
def test_quant_validation(lib, fn):
    src, q, s = A, 64 * A, 128 * A
    assert _q(lib, fn, None, 4, 64, 64, q, s) == ENULL
    assert _q(lib, fn, src, 4, 64, 64, None, s) == ENULL
    assert _q(lib, fn, src, 4, 64, 64, q, None) == ENULL
    assert _q(lib, fn, src, -1, 64, 64, q, s) == ESHAPE
    assert _q(lib, fn, src, 4, 0, 64, q, s) == ESHAPE
    assert _q(lib, fn, src, 4, 60, 64, q, s) == ESHAPE       # k % 8
    assert _q(lib, fn, src, 4, 64, 32, q, s) == ESHAPE       # ld < k
    assert _q(lib, fn, src, 4, 64, 68, q, s) == ESHAPE       # ld % 8
    assert _q(lib, fn, src + 8, 4, 64, 64, q, s) == EALIGN
    assert _q(lib, fn, src, 4, 64, 64, q + 4, s) == EALIGN
    assert _q(lib, fn, src, 4, 64, 64, q, s + 2) == EALIGN
    assert _q(lib, fn, src, 4, 64, 64, src + 64, s) == EALIAS  # q inside x
    assert _q(lib, fn, src, 4, 64, 64, q, q + 16) == EALIAS    # s inside q
    # empty is a valid no-op and needs no device
    assert _q(lib, fn, src, 0, 64, 64, q, s) == OK


def _norm(lib, x=A, m=4, k=64, ldx=64, g=2 * A, eps=1e-6, q=64 * A, s=128 * A,
          y=256 * A, ldy=64):
    return lib.fp8w8a8_rmsnorm_quantize(x, m, k, ldx, g, eps, q, s, y, ldy, None)


def test_rmsnorm_quantize_validation(lib):
    assert _norm(lib, x=None) == ENULL
    assert _norm(lib, g=None) == ENULL
    assert _norm(lib, q=None) == ENULL
    assert _norm(lib, s=None) == ENULL
    assert _norm(lib, m=-1) == ESHAPE
    assert _norm(lib, k=0) == ESHAPE
    assert _norm(lib, k=60, ldx=64, ldy=64) == ESHAPE      # k % 8
    assert _norm(lib, ldx=32) == ESHAPE                     # ldx < k
    assert _norm(lib, ldx=68) == ESHAPE                     # ldx % 8
    assert _norm(lib, ldy=32) == ESHAPE                     # ldy < k
    assert _norm(lib, ldy=72 + 4) == ESHAPE                 # ldy % 8
    for eps in (-1e-6, float("nan"), float("inf")):
        assert _norm(lib, eps=eps) == ESHAPE
    assert _norm(lib, x=A + 8) == EALIGN
    assert _norm(lib, g=2 * A + 8) == EALIGN
    assert _norm(lib, q=64 * A + 4) == EALIGN
    assert _norm(lib, y=256 * A + 2) == EALIGN
    assert _norm(lib, s=128 * A + 2) == EALIGN
    assert _norm(lib, q=A + 64) == EALIAS                   # codes inside x
    assert _norm(lib, s=2 * A) == EALIAS                    # scales over gamma
    assert _norm(lib, y=64 * A + 128) == EALIAS             # y inside codes
    assert _norm(lib, s=256 * A + 16) == EALIAS             # scales inside y
    # empty is a valid no-op and needs no device, with or without y
    assert _norm(lib, m=0) == OK
    assert _norm(lib, m=0, y=None, ldy=0) == OK


def _swi(lib, g=A, ldg=128, u=A + 128, ldu=128, m=4, n=64, q=64 * A, s=128 * A,
         h=256 * A, ldh=64):
    return lib.fp8w8a8_swiglu_quantize(g, ldg, u, ldu, m, n, q, s, h, ldh, None)


def test_swiglu_quantize_validation(lib):
    assert _swi(lib, g=None) == ENULL
    assert _swi(lib, u=None) == ENULL
    assert _swi(lib, q=None) == ENULL
    assert _swi(lib, s=None) == ENULL
    assert _swi(lib, m=-1) == ESHAPE
    assert _swi(lib, n=0) == ESHAPE
    assert _swi(lib, n=60, ldh=64) == ESHAPE                 # n % 8
    assert _swi(lib, ldg=32) == ESHAPE
    assert _swi(lib, ldu=132) == ESHAPE
    assert _swi(lib, ldh=32) == ESHAPE
    assert _swi(lib, g=A + 8) == EALIGN
    assert _swi(lib, u=A + 136) == EALIGN
    assert _swi(lib, q=64 * A + 8) == EALIGN
    assert _swi(lib, h=256 * A + 4) == EALIGN
    assert _swi(lib, s=128 * A + 1) == EALIGN
    assert _swi(lib, q=A + 256) == EALIAS                    # codes over gate/up rows
    assert _swi(lib, h=64 * A + 64) == EALIAS                # h over codes
    assert _swi(lib, s=256 * A) == EALIAS                    # scales over h
    assert _swi(lib, m=0) == OK
    assert _swi(lib, m=0, h=None, ldh=0) == OK


def _kvq(lib, x=A, t=4, w=1024, ld=1024, g=128, c=64 * A, s=128 * A):
    return lib.fp8w8a8_kv_quantize_fp8(x, t, w, ld, g, c, s, None)


def _kvd(lib, c=A, s=2 * A, t=4, w=1024, g=128, o=64 * A, ldo=1024):
    return lib.fp8w8a8_kv_dequantize_fp8(c, s, t, w, g, o, ldo, None)


def test_kv_codec_validation(lib):
    assert _kvq(lib, x=None) == ENULL
    assert _kvq(lib, c=None) == ENULL
    assert _kvq(lib, s=None) == ENULL
    assert _kvq(lib, t=-1) == ESHAPE
    assert _kvq(lib, w=4, ld=8, g=8) == ESHAPE
    for g in (0, 4, 96, 1024, 48):
        assert _kvq(lib, g=g) == ESHAPE                       # power of two, 8..512
    assert _kvq(lib, w=1000, ld=1000, g=16) == ESHAPE         # 1000 % 16
    assert _kvq(lib, ld=1000) == ESHAPE
    assert _kvq(lib, x=A + 8) == EALIGN
    assert _kvq(lib, c=64 * A + 4) == EALIGN
    assert _kvq(lib, s=128 * A + 2) == EALIGN
    assert _kvq(lib, c=A + 4096) == EALIAS                    # codes inside kv
    assert _kvq(lib, s=64 * A + 512) == EALIAS                # scales inside codes
    assert _kvq(lib, t=0) == OK
    assert _kvd(lib, c=None) == ENULL
    assert _kvd(lib, o=None) == ENULL
    assert _kvd(lib, g=12) == ESHAPE
    assert _kvd(lib, ldo=1020) == ESHAPE
    assert _kvd(lib, o=64 * A + 8) == EALIGN
    assert _kvd(lib, c=A + 4) == EALIGN
    assert _kvd(lib, o=A + 16) == EALIAS                      # out over codes
    assert _kvd(lib, t=0) == OK


def test_kv_int8_validation(lib):
    q = lambda **k: lib.fp8w8a8_kv_quantize_int8(
        k.get("x", A), k.get("t", 4), k.get("w", 1024), k.get("ld", 1024), k.get("g", 64),
        k.get("c", 64 * A), k.get("s", 128 * A), k.get("m", 192 * A), None)
    assert q(x=None) == ENULL and q(m=None) == ENULL
    assert q(g=48) == ESHAPE and q(g=1024) == ESHAPE and q(ld=1020) == ESHAPE
    assert q(m=192 * A + 2) == EALIGN
    assert q(m=128 * A + 32) == EALIAS                        # mins over scales
    assert q(t=0) == OK
    r = lambda **k: lib.fp8w8a8_kv_read_int8(
        k.get("c", A), k.get("s", 2 * A), k.get("m", 3 * A), k.get("h", 4),
        k.get("tl", 64 * A), k.get("tr", 2), k.get("ldt", 1024), k.get("w", 1024),
        k.get("g", 64), k.get("o", 128 * A), k.get("ldo", 1024), None)
    assert r(o=None) == ENULL
    assert r(c=None) == ENULL and r(tl=None) == ENULL
    assert r(c=None, s=None, m=None, h=0, o=128 * A, tr=0, tl=None) == OK   # empty
    assert r(h=-1) == ESHAPE and r(ldt=1000) == ESHAPE and r(g=24) == ESHAPE
    assert r(tl=64 * A + 8) == EALIGN
    assert r(o=64 * A) == EALIAS                              # out over the tail
    assert r(c=None, s=None, m=None, h=0, tr=0, tl=None, o=128 * A + 8) == EALIGN


def test_pre_linear_validation(lib):
    nrm = lambda **k: lib.fp8w8a8_rmsnorm_quant_linear(
        k.get("x", A), k.get("ldx", 256), k.get("g", 2 * A), k.get("eps", 1e-6),
        k.get("qw", 4 * A), k.get("sw", 8 * A), k.get("m", 32), k.get("n", 64),
        k.get("k", 256), k.get("y", 16 * A), k.get("ldy", 64), k.get("ws", None),
        k.get("wsb", 0), None)
    assert nrm(x=None) == ENULL and nrm(g=None) == ENULL
    assert nrm(k=192, ldx=192) == ESHAPE                       # k % 128
    assert nrm(n=24) == ESHAPE
    assert nrm(ldx=200) == ESHAPE
    assert nrm(eps=-1.0) == ESHAPE and nrm(eps=float("nan")) == ESHAPE
    assert nrm(g=2 * A + 8) == EALIGN
    assert nrm(y=A + 512) == EALIAS                            # y over x
    assert nrm(y=2 * A) == EALIAS                              # y over gamma
    assert nrm() == EWS                                        # m = 32 needs a workspace
    assert nrm(m=0) == EWS or nrm(m=0, ws=64 * A, wsb=1 << 20) == OK
    swi = lambda **k: lib.fp8w8a8_swiglu_quant_linear(
        k.get("g", A), k.get("ldg", 256), k.get("u", 2 * A), k.get("ldu", 256),
        k.get("qw", 4 * A), k.get("sw", 8 * A), k.get("m", 32), k.get("n", 64),
        k.get("k", 256), k.get("y", 16 * A), k.get("ldy", 64), k.get("ws", None),
        k.get("wsb", 0), None)
    assert swi(u=None) == ENULL
    assert swi(ldu=200) == ESHAPE
    assert swi(u=2 * A + 4) == EALIGN
    assert swi(y=2 * A + 256) == EALIAS                        # y over up
    assert swi() == EWS
    ws_norm = lib.fp8w8a8_workspace_bytes(32, 64, 256, 2)
    assert ws_norm == lib.fp8w8a8_workspace_bytes(32, 64, 256, 1) > 0
    assert lib.fp8w8a8_workspace_bytes(2, 4096, 4096, 2) == 0   # fused into the GEMV
    # one token: norm kernel, then the barrier-free M = 1 GEMV on its codes
    assert lib.fp8w8a8_workspace_bytes(1, 4096, 4096, 2) >= 4096 + 4
    assert lib.fp8w8a8_workspace_bytes(1, 4096, 4224, 2) > 0    # k % 512 != 0
    assert lib.fp8w8a8_workspace_bytes(1, 4096, 4224, 3) == 0
    assert lib.fp8w8a8_workspace_bytes(2, 4096, 12288, 3) > 0   # m * k too large


def _lin(lib, qx=A, sx=2 * A, qw=4 * A, sw=8 * A, m=32, n=64, k=256,
         y=16 * A, ldy=64, ws=None, wsb=0):
    return lib.fp8w8a8_fp8_linear(qx, sx, qw, sw, m, n, k, y, ldy, ws, wsb, None)


def test_linear_validation(lib):
    assert _lin(lib, qx=None) == ENULL
    assert _lin(lib, y=None) == ENULL
    assert _lin(lib, n=24) == ESHAPE            # n % 16
    assert _lin(lib, k=192) == ESHAPE           # k % 128
    assert _lin(lib, k=0) == ESHAPE
    assert _lin(lib, k=(1 << 22) + 128) == ESHAPE   # beyond 32-bit tile offsets
    assert _lin(lib, m=-1) == ESHAPE
    assert _lin(lib, ldy=32) == ESHAPE          # ldy < n
    assert _lin(lib, ldy=68) == ESHAPE          # ldy % 8
    assert _lin(lib, qw=4 * A + 8) == EALIGN
    assert _lin(lib, y=A + 64) == EALIAS        # y overlaps qx
    assert _lin(lib, m=0) == OK
    assert _lin(lib, n=0) == OK
    # the pre-quantized linear needs scratch only where the GEMM splits K
    # (few output tiles: float32 partial sums of at least two splits)
    assert lib.fp8w8a8_workspace_bytes(1, 64, 4096, 0) == 0
    assert lib.fp8w8a8_workspace_bytes(16, 4096, 4096, 0) == 0
    assert lib.fp8w8a8_workspace_bytes(4096, 4096, 4096, 0) == 0
    assert lib.fp8w8a8_workspace_bytes(64, 4096, 4096, 0) >= 2 * 64 * 4096 * 4
    assert lib.fp8w8a8_workspace_bytes(64, 4096, 12288, 0) >= 2 * 64 * 4096 * 4


def _req(lib, qx=A, sx=2 * A, qw=4 * A, sw=24 * A, m=64, n=4096, k=4096, y=32 * A,
         ldy=4096, qy=40 * A, sy=44 * A, ws=48 * A, wsb=1 << 24):
    # qw spans 16 MiB from 4 A; every other buffer fits in its 1-8 MiB slot
    return lib.fp8w8a8_fp8_linear_requant(qx, sx, qw, sw, m, n, k, y, ldy, qy, sy, ws,
                                          wsb, None)


def test_linear_requant_validation(lib):
    assert _req(lib, qy=None) == ENULL
    assert _req(lib, sy=None) == ENULL
    assert _req(lib, y=None) == ENULL
    assert _req(lib, n=24) == ESHAPE            # n % 16
    assert _req(lib, k=192) == ESHAPE           # k % 128
    assert _req(lib, ldy=4088) == ESHAPE        # ldy < n
    assert _req(lib, qy=40 * A + 8) == EALIGN
    assert _req(lib, sy=44 * A + 2) == EALIGN
    assert _req(lib, qy=32 * A + 64) == EALIAS  # codes inside y
    assert _req(lib, sy=40 * A + 64) == EALIAS  # scales inside the codes
    assert _req(lib, sy=32 * A) == EALIAS       # scales inside y
    assert _req(lib, qy=A) == EALIAS            # codes over the input codes
    assert _req(lib, sy=24 * A) == EALIAS       # scales over the weight scales
    assert _req(lib, y=8 * A) == EALIAS         # y inside the weight codes
    # m = 64, k = 12288: the GEMM splits K, so the partial sums need the
    # workspace, which must not overlap any output (qw: 12 MiB from 4 A)
    long_k = dict(n=1024, k=12288, ldy=1024)
    assert _req(lib, **long_k) == EDEV
    assert _req(lib, ws=None, wsb=0, **long_k) == EWS
    assert _req(lib, wsb=1024, **long_k) == EWS
    assert _req(lib, ws=40 * A, **long_k) == EALIAS
    assert _req(lib, m=0) == OK
    assert _req(lib, n=0) == OK


def test_quant_linear_validation(lib):
    f = lib.fp8w8a8_quant_linear
    args = dict(x=A, ldx=256, qw=4 * A, sw=8 * A, m=64, n=64, k=256, y=16 * A,
                ldy=64, ws=32 * A, wsb=1 << 30)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["x"], a["ldx"], a["qw"], a["sw"], a["m"], a["n"], a["k"],
                 a["y"], a["ldy"], a["ws"], a["wsb"], None)

    assert call(x=None) == ENULL
    assert call(ldx=128) == ESHAPE
    assert call(ldx=260) == ESHAPE
    assert call(sw=8 * A + 4) == EALIGN
    assert call(y=A + 32) == EALIAS
    assert call(ws=None, wsb=0) == EWS
    assert call(ws=A, wsb=1 << 30) == EALIAS
    assert call(m=0) == OK


def test_workspace_sizes(lib):
    fused = lib.fp8w8a8_workspace_bytes(4096, 4096, 4096, 1)
    assert fused >= 4096 * 4096 + 4 * 4096                       # qx + sx
    # decode-sized fused calls quantize inside the GEMV kernel: no scratch
    assert lib.fp8w8a8_workspace_bytes(1, 4096, 4096, 1) == 0
    # ... unless the codes do not fit the kernel's LDS copy
    assert lib.fp8w8a8_workspace_bytes(16, 4096, 12288, 1) >= 16 * 12288
    assert lib.fp8w8a8_workspace_bytes(1, 24, 4096, 0) == 0      # invalid n
    assert lib.fp8w8a8_workspace_init(None, 16, None) == ENULL
    assert lib.fp8w8a8_workspace_init(A, 8, None) == ESHAPE
    assert lib.fp8w8a8_workspace_init(A + 8, 16, None) == EALIGN
    assert lib.fp8w8a8_workspace_init(A, 0, None) == OK


def test_peaks_library_exports_and_validates():
    """The benchmark's measured-peak library: every symbol its header
    declares is exported, and bad arguments are refused before a launch."""
    from fp8_w8a8_dynamic_amd import build as fbuild
    text = open(os.path.join(ROOT, "include", "fp8w8a8_peaks.h")).read()
    names = sorted(set(re.findall(r"\b(fp8w8a8_[a-z_0-9]+)\s*\(", text)))
    assert len(names) == 5
    plib = ctypes.CDLL(fbuild.PEAKS_LIB_PATH)
    for name in names:
        assert hasattr(plib, name), name
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    plib.fp8w8a8_peaks_mfma_flops.restype = i64
    plib.fp8w8a8_peaks_mfma_flops.argtypes = [i64, ctypes.c_int]
    assert plib.fp8w8a8_peaks_mfma_flops(2048, 2048) == 2048 * 4 * 8 * 2048 * 131072
    plib.fp8w8a8_peaks_read_workgroups.restype = i64
    plib.fp8w8a8_peaks_read_workgroups.argtypes = [i64]
    assert plib.fp8w8a8_peaks_read_workgroups(2 << 30) == 1024
    plib.fp8w8a8_peaks_mfma_loop.argtypes = [vp, vp, i64, ctypes.c_int, vp]
    plib.fp8w8a8_peaks_read_stream.argtypes = [vp, i64, vp, vp]
    assert plib.fp8w8a8_peaks_mfma_loop(None, A, 4, 4, None) == 1
    assert plib.fp8w8a8_peaks_mfma_loop(A, A, 0, 4, None) == 2
    assert plib.fp8w8a8_peaks_mfma_loop(A, A, 4, 0, None) == 2
    assert plib.fp8w8a8_peaks_read_stream(None, 1024, A, None) == 1
    assert plib.fp8w8a8_peaks_read_stream(A, 1000, A, None) == 2
    assert plib.fp8w8a8_peaks_read_stream(A + 8, 1024, A, None) == 3


BIG = 1 << 31        # one past the largest row stride (2^31 - 1 elements)


def test_strides_are_bounded(lib):
    """Every row stride is bounded by 2^31 - 1 elements, so the byte ranges
    of the overlap checks cannot wrap around the address space."""
    assert _q(lib, "fp8w8a8_quantize_act_per_token", A, 4, 64, BIG, 64 * A, 128 * A) == ESHAPE
    assert _q(lib, "fp8w8a8_quantize_act_per_token", A, 4, 64, BIG - 8, 64 * A, 128 * A) \
        in (EALIAS, EDEV)      # in range: x now spans the other buffers' addresses
    assert _norm(lib, ldx=BIG) == ESHAPE
    assert _norm(lib, ldy=BIG) == ESHAPE
    assert _swi(lib, ldg=BIG) == ESHAPE and _swi(lib, ldu=BIG) == ESHAPE
    assert _swi(lib, ldh=BIG) == ESHAPE
    assert _kvq(lib, ld=BIG) == ESHAPE and _kvd(lib, ldo=BIG) == ESHAPE
    assert _lin(lib, ldy=BIG) == ESHAPE
    f = lib.fp8w8a8_quant_linear
    assert f(A, BIG, 4 * A, 8 * A, 64, 64, 256, 16 * A, 64, 32 * A, 1 << 30, None) == ESHAPE
    assert lib.fp8w8a8_rmsnorm_quant_linear(A, BIG, 2 * A, 1e-6, 4 * A, 8 * A, 32, 64, 256,
                                            16 * A, 64, None, 0, None) == ESHAPE
    assert lib.fp8w8a8_swiglu_quant_linear(A, 256, 2 * A, BIG, 4 * A, 8 * A, 32, 64, 256,
                                           16 * A, 64, None, 0, None) == ESHAPE
    # the largest valid stride and row count: the range saturates at the top
    # of the address space instead of wrapping, so the overlap test still
    # sees y reaching over the workspace placed after it
    hi = (1 << 63) - (1 << 40)
    assert f(A, 256, 4 * A, 8 * A, BIG - 1, 64, 256, hi, BIG - 8, hi + (1 << 30), 1 << 62,
             None) == EALIAS


def test_overrides_off_without_the_test_switch():
    """The tuning overrides are honoured only with FP8W8A8_TEST_HOOKS=1 set
    when the library first looks: a fresh process without the switch and
    with an override that would change the workspace size gets the
    production plan."""
    import subprocess
    import sys
    code = (
        "from fp8_w8a8_dynamic_amd import load_library\n"
        "lib = load_library()\n"
        "print(lib.fp8w8a8_workspace_bytes(1, 64, 4096, 0),"
        " lib.fp8w8a8_workspace_bytes(64, 4096, 4096, 0))\n")
    outs = {}
    for hooks in ("0", "1"):
        env = dict(os.environ, FP8W8A8_TEST_HOOKS=hooks, FP8W8A8_FORCE_PATH="gemm",
                   FP8W8A8_GEMM_CONFIG="5", FP8W8A8_GEMM_SPLITS="2")
        lib_env = os.environ.get("FP8W8A8_ABI_TEST_LIBRARY")
        if lib_env:
            code_run = code.replace("load_library()", f"load_library({lib_env!r})")
        else:
            code_run = code
        res = subprocess.run([sys.executable, "-c", code_run], env=env, cwd=ROOT,
                             capture_output=True, text=True, timeout=300)
        assert res.returncode == 0, res.stderr[-2000:]
        outs[hooks] = [int(v) for v in res.stdout.split()]
    assert outs["0"][0] == 0                      # M = 1 stays on the GEMV: no scratch
    assert outs["1"][0] == 2 * 1 * 64 * 4         # forced 2-way split-K GEMM
    assert outs["0"][1] != outs["1"][1]


def test_quant_linear_noalloc_validation(lib):
    """The allocation-free fused entry point validates like quant_linear and
    refuses, before touching a device, a call whose staging would not fit
    its fixed scratch array (64 MiB)."""
    f = lib.fp8w8a8_quant_linear_noalloc
    assert f(None, 256, 4 * A, 8 * A, 64, 64, 256, 16 * A, 64, None) == ENULL
    assert f(A, 256, 4 * A, 8 * A, 64, 24, 256, 16 * A, 64, None) == ESHAPE
    assert f(A, BIG, 4 * A, 8 * A, 64, 64, 256, 16 * A, 64, None) == ESHAPE
    assert f(A + 8, 256, 4 * A, 8 * A, 64, 64, 256, 16 * A, 64, None) == EALIGN
    assert f(A, 256, 4 * A, 8 * A, 64, 64, 256, A + 64, 64, None) == EALIAS
    # 16384 x 4096 codes + scales: 64 MiB + 64 KiB of staging > 64 MiB
    assert lib.fp8w8a8_workspace_bytes(16384, 4096, 4096, 1) > 64 << 20
    assert f(A, 4096, 4 * A, 8 * A, 16384, 4096, 4096, 1 << 40, 4096, None) == EWS
    # 16000 rows fit
    assert lib.fp8w8a8_workspace_bytes(16000, 4096, 4096, 1) <= 64 << 20
    assert f(A, 4096, 4 * A, 8 * A, 16000, 4096, 4096, 1 << 40, 4096, None) == EDEV
    assert f(A, 256, 4 * A, 8 * A, 0, 64, 256, 16 * A, 64, None) == OK


def test_group_m1_validation(lib):
    """The grouped one-token call validates every item before a launch."""
    from fp8_w8a8_dynamic_amd.binding import _GroupLinear

    def run(items):
        arr = (_GroupLinear * max(1, len(items)))(*items)
        return lib.fp8w8a8_quant_linear_group_m1(arr, len(items), None)

    def item(x=A, qw=4 * A, sw=8 * A, y=16 * A, n=64, k=256):
        return _GroupLinear(x, qw, sw, y, n, k)

    assert lib.fp8w8a8_quant_linear_group_m1(None, 1, None) == ENULL
    assert run([]) == ESHAPE                                    # count 0
    assert run([item()] * 17) == ESHAPE                         # count > 16
    assert run([item(x=None)]) == ENULL
    assert run([item(n=24)]) == ESHAPE and run([item(n=0)]) == ESHAPE
    assert run([item(k=192)]) == ESHAPE
    assert run([item(k=12288 + 128)]) == ESHAPE                 # K <= 12288
    assert run([item(y=16 * A + 8)]) == EALIGN
    assert run([item(y=A + 64)]) == EALIAS                      # y over its x
    assert run([item(), item(x=32 * A, y=16 * A + 64)]) == EALIAS   # ys overlap
    assert run([item(), item(x=16 * A, y=64 * A)]) == EALIAS    # y over another x
    assert run([item(), item(x=32 * A, y=64 * A)]) == EDEV      # valid: no device here


def test_quantize_act_group_validation(lib):
    """The grouped quantizer validates every item and the cross-item
    overlaps before a launch."""
    from fp8_w8a8_dynamic_amd.binding import _GroupQuant

    def run(items):
        arr = (_GroupQuant * max(1, len(items)))(*items)
        return lib.fp8w8a8_quantize_act_group(arr, len(items), None)

    def item(x=A, m=4, k=256, ldx=256, qx=8 * A, sx=16 * A):
        return _GroupQuant(x, m, k, ldx, qx, sx)

    assert lib.fp8w8a8_quantize_act_group(None, 1, None) == ENULL
    assert run([]) == ESHAPE and run([item()] * 17) == ESHAPE
    assert run([item(x=None)]) == ENULL and run([item(sx=None)]) == ENULL
    assert run([item(k=12)]) == ESHAPE                          # k % 8
    assert run([item(k=16384 + 8, ldx=16392)]) == ESHAPE        # k <= 16384
    assert run([item(ldx=128)]) == ESHAPE                       # ldx < k
    assert run([item(m=-1)]) == ESHAPE
    assert run([item(qx=8 * A + 8)]) == EALIGN
    assert run([item(qx=A + 512)]) == EALIAS                    # codes over its x
    # Codes of one item over another item's input, or over its codes.
    assert run([item(), item(x=32 * A, qx=32 * A + 256, sx=48 * A)]) == EALIAS
    assert run([item(), item(x=32 * A, qx=8 * A + 512, sx=48 * A)]) == EALIAS
    assert run([item(), item(x=32 * A, qx=A + 256, sx=48 * A)]) == EALIAS  # over item 0's x
    assert run([item(m=0), item(m=0, x=32 * A, qx=40 * A, sx=48 * A)]) == OK   # empty
    assert run([item(m=0, x=None, qx=None, sx=None)]) == OK     # empty: no pointers needed
    assert run([item(m=0, k=12, x=None, qx=None, sx=None)]) == ESHAPE
    assert run([item(), item(x=32 * A, qx=40 * A, sx=48 * A)]) == EDEV          # valid


def test_tile_weights_validation(lib):
    f = lib.fp8w8a8_tile_weights
    assert f(None, 16, 128, A, None) == ENULL and f(A, 16, 128, None, None) == ENULL
    assert f(A, 24, 128, 4 * A, None) == ESHAPE                 # n % 16
    assert f(A, 16, 192, 4 * A, None) == ESHAPE                 # k % 128
    assert f(A, 16, 16384 + 128, 4 * A, None) == ESHAPE         # k <= 16384
    assert f(A, -16, 128, 4 * A, None) == ESHAPE
    assert f(A + 8, 16, 128, 4 * A, None) == EALIGN
    assert f(A, 16, 128, A + 1024, None) == EALIAS              # ranges overlap
    assert f(A, 0, 128, 4 * A, None) == OK                      # empty
    assert f(A, 16, 128, 4 * A, None) == EDEV                   # valid: no device here


def test_fp8_linear_group_validation(lib):
    """The grouped call on given codes validates m and every item before a
    launch."""
    from fp8_w8a8_dynamic_amd.binding import _GroupFp8Linear

    def run(items, m=64):
        arr = (_GroupFp8Linear * max(1, len(items)))(*items)
        return lib.fp8w8a8_fp8_linear_group(arr, len(items), m, None)

    def item(qx=A, sx=2 * A, qw=4 * A, sw=8 * A, y=16 * A, n=128, k=256):
        return _GroupFp8Linear(qx, sx, qw, sw, y, n, k)

    assert lib.fp8w8a8_fp8_linear_group(None, 1, 64, None) == ENULL
    assert run([]) == ESHAPE                                    # count 0
    assert run([item()] * 17) == ESHAPE                         # count > 16
    assert run([item()], m=0) == ESHAPE and run([item()], m=257) == ESHAPE
    assert run([item(n=(1 << 24))], m=64) != ESHAPE              # m * n = 2^30
    assert run([item(n=(1 << 24))], m=65) == ESHAPE              # m * n > 2^30
    assert run([item(sx=None)]) == ENULL and run([item(qw=None)]) == ENULL
    assert run([item(n=96)]) == ESHAPE and run([item(n=0)]) == ESHAPE
    assert run([item(n=(1 << 24) + 64)]) == ESHAPE              # n <= 2^24
    assert run([item(k=192)]) == ESHAPE and run([item(k=64)]) == ESHAPE
    assert run([item(k=16384 + 128)]) == ESHAPE                 # k <= 16384
    assert run([item(sx=2 * A + 4)]) == EALIGN
    assert run([item(y=A + 64)]) == EALIAS                      # y over its codes
    assert run([item(y=2 * A)]) == EALIAS                       # y over its scales
    assert run([item(y=4 * A + 64)]) == EALIAS                  # y over its weights
    # ys of 64 x 128 bf16 (16 KB): overlapping, and over another item's codes.
    assert run([item(), item(y=16 * A + 8192)]) == EALIAS
    assert run([item(), item(qx=16 * A, y=64 * A)]) == EALIAS
    # Valid, with the codes shared by both items: no device here.
    assert run([item(), item(qw=32 * A, sw=48 * A, y=64 * A)]) == EDEV
    assert run([item(n=64, k=128)], m=1) == EDEV


def test_fp8_linear_group_requant_validation(lib):
    """The grouped call with one item re-quantized: the items' rules, rq in
    range with n <= 16384, the extra outputs' alignment and overlaps, and
    the workspace, all checked before a launch; the workspace query gives
    ranges x m x n x 4 bytes, 0 for invalid arguments."""
    from fp8_w8a8_dynamic_amd.binding import _GroupFp8Linear

    def arr(items):
        return (_GroupFp8Linear * max(1, len(items)))(*items)

    def ws_bytes(items, m=64, rq=0):
        return lib.fp8w8a8_group_requant_workspace_bytes(arr(items), len(items), m, rq)

    def run(items, m=64, rq=0, qy=80 * A, sy=96 * A, ws=112 * A, wsb=1 << 24):
        return lib.fp8w8a8_fp8_linear_group_requant(arr(items), len(items), m, rq, qy, sy,
                                                    ws, wsb, None)

    # A is 1 MiB: down's weights (48 MiB) at 1024 A, k's and v's (4 MiB
    # each) at 1100 A and 1110 A.
    def item(qx=A, sx=2 * A, qw=1024 * A, sw=8 * A, y=16 * A, n=4096, k=12288):
        return _GroupFp8Linear(qx, sx, qw, sw, y, n, k)

    down = item()
    kv = [item(qx=128 * A, sx=130 * A, qw=1100 * A, sw=134 * A, y=136 * A, n=1024, k=4096),
          item(qx=128 * A, sx=130 * A, qw=1110 * A, sw=142 * A, y=144 * A, n=1024, k=4096)]
    # Down alone (64 units): the most 512-byte-stage ranges that keep the
    # launch at one workgroup per CU (256) is 4; beside k and v (32 units),
    # 3 (3 x 64 + 32 <= 256).
    assert ws_bytes([down]) == 4 * 64 * 4096 * 4
    assert ws_bytes([down] + kv) == 3 * 64 * 4096 * 4
    assert ws_bytes(kv + [down], rq=2) == 3 * 64 * 4096 * 4
    assert ws_bytes([down], m=3) == 4 * 3 * 4096 * 4
    assert ws_bytes([down], rq=1) == 0 and ws_bytes([down], rq=-1) == 0
    # n > 16384 is allowed without re-quantization (checked at the call);
    # its 257 units alone exceed one per CU, so one range.
    assert ws_bytes([item(n=16384 + 64)]) == 64 * (16384 + 64) * 4
    # Beside items of K = 4096: ranges no shorter than 4096 (decode layer).
    assert ws_bytes([down, item(qx=300 * A, sx=302 * A, qw=1300 * A, sw=304 * A,
                                y=306 * A, n=12288, k=4096)], m=4) == 3 * 4 * 4096 * 4
    assert ws_bytes([item(n=96)]) == 0
    assert lib.fp8w8a8_group_requant_workspace_bytes(None, 1, 64, 0) == 0
    # K = 640: 5 tiles, no split into whole stages (one range).
    assert ws_bytes([item(k=640)]) == 64 * 4096 * 4

    assert lib.fp8w8a8_fp8_linear_group_requant(None, 1, 64, 0, 80 * A, 96 * A, 112 * A,
                                                1 << 24, None) == ENULL
    assert run([]) == ESHAPE and run([down] * 17) == ESHAPE
    assert run([down], m=0) == ESHAPE and run([down], m=257) == ESHAPE
    assert run([down], rq=1) == ESHAPE and run([down], rq=-1) == ESHAPE
    assert run([item(n=16384 + 64)]) == ESHAPE
    assert run([item(sx=None)]) == ENULL
    assert run([down], qy=None) == ENULL and run([down], sy=None) == ENULL
    # Both null: the ranges added without re-quantization (no n limit).
    assert run([down], qy=None, sy=None) == EDEV
    assert run([item(n=16384 + 64)], qy=None, sy=None) == EDEV
    # The split item's sums are addressed in 32 bits: n <= 2^20.
    big = item(qw=4096 * A, y=64 * A, n=(1 << 20) + 64, k=128)
    assert ws_bytes([big]) == 0
    assert run([big], qy=None, sy=None, ws=8192 * A) == ESHAPE
    assert run([down], qy=None, sy=None, ws=None) == ENULL
    assert run([down], qy=None, sy=None, wsb=4 * 64 * 4096 * 4 - 1) == EWS
    assert run([down], qy=None, sy=None, ws=1030 * A) == EALIAS
    assert run([down], ws=None) == ENULL
    assert run([down], qy=80 * A + 8) == EALIGN and run([down], sy=96 * A + 2) == EALIGN
    assert run([down], ws=112 * A + 8) == EALIGN
    assert run([down], wsb=4 * 64 * 4096 * 4 - 1) == EWS
    assert run([down], qy=A + 64) == EALIAS                     # qy over the codes
    assert run([down], sy=16 * A + 4) == EALIAS                 # scales over y
    assert run([down], ws=1030 * A) == EALIAS                   # workspace over weights
    assert run([down], qy=112 * A + 4096) == EALIAS             # qy in the workspace
    assert run([down] + kv, qy=136 * A) == EALIAS               # qy over k's y
    # Item rules are the grouped call's (y over another item's codes).
    assert run([down, item(qx=16 * A, qw=1200 * A, sw=202 * A, y=204 * A, n=64, k=128)]) \
        == EALIAS
    # Valid: no device here.
    assert run([down]) == EDEV and run([down] + kv) == EDEV
    assert run(kv + [down], rq=2) == EDEV
