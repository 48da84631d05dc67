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
    return load_library()


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert len(names) == 16
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
    assert lib.fp8w8a8_workspace_bytes(1, 4096, 4096, 2) == 0   # fused into the GEMV
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
