"""Thin ctypes binding of ``libfp8w8a8.so`` (the C ABI in include/fp8w8a8.h).

The functions here only marshal torch tensors into pointers, sizes and the
current HIP stream; every step of the computation runs in the library's HIP
kernels.  If the library is missing or fails to load, every call raises:
there is no fallback path.
"""

import ctypes
import os
import threading

import torch

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIBRARY_PATH = os.path.join(_PKG_DIR, "libfp8w8a8.so")

_c_i64 = ctypes.c_int64
_c_vp = ctypes.c_void_p
_c_sz = ctypes.c_size_t

#: exported symbol -> (restype, argtypes), mirroring include/fp8w8a8.h
SIGNATURES = {
    "fp8w8a8_quantize_weight_channelwise":
        (ctypes.c_int, [_c_vp, _c_i64, _c_i64, _c_i64, _c_vp, _c_vp, _c_vp]),
    "fp8w8a8_quantize_act_per_token":
        (ctypes.c_int, [_c_vp, _c_i64, _c_i64, _c_i64, _c_vp, _c_vp, _c_vp]),
    "fp8w8a8_rmsnorm_quantize":
        (ctypes.c_int, [_c_vp, _c_i64, _c_i64, _c_i64, _c_vp, ctypes.c_float,
                        _c_vp, _c_vp, _c_vp, _c_i64, _c_vp]),
    "fp8w8a8_swiglu_quantize":
        (ctypes.c_int, [_c_vp, _c_i64, _c_vp, _c_i64, _c_i64, _c_i64, _c_vp,
                        _c_vp, _c_vp, _c_i64, _c_vp]),
    "fp8w8a8_kv_quantize_fp8":
        (ctypes.c_int, [_c_vp, _c_i64, _c_i64, _c_i64, _c_i64, _c_vp, _c_vp, _c_vp]),
    "fp8w8a8_kv_dequantize_fp8":
        (ctypes.c_int, [_c_vp, _c_vp, _c_i64, _c_i64, _c_i64, _c_vp, _c_i64, _c_vp]),
    "fp8w8a8_kv_quantize_int8":
        (ctypes.c_int, [_c_vp, _c_i64, _c_i64, _c_i64, _c_i64, _c_vp, _c_vp, _c_vp,
                        _c_vp]),
    "fp8w8a8_kv_read_int8":
        (ctypes.c_int, [_c_vp, _c_vp, _c_vp, _c_i64, _c_vp, _c_i64, _c_i64, _c_i64,
                        _c_i64, _c_vp, _c_i64, _c_vp]),
    "fp8w8a8_fp8_linear":
        (ctypes.c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64,
                        _c_vp, _c_i64, _c_vp, _c_sz, _c_vp]),
    "fp8w8a8_fp8_linear_requant":
        (ctypes.c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64,
                        _c_vp, _c_i64, _c_vp, _c_vp, _c_vp, _c_sz, _c_vp]),
    "fp8w8a8_quant_linear":
        (ctypes.c_int, [_c_vp, _c_i64, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64,
                        _c_vp, _c_i64, _c_vp, _c_sz, _c_vp]),
    "fp8w8a8_quant_linear_noalloc":
        (ctypes.c_int, [_c_vp, _c_i64, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64,
                        _c_vp, _c_i64, _c_vp]),
    "fp8w8a8_quant_linear_group_m1":
        (ctypes.c_int, [_c_vp, ctypes.c_int, _c_vp]),
    "fp8w8a8_quantize_act_group":
        (ctypes.c_int, [_c_vp, ctypes.c_int, _c_vp]),
    "fp8w8a8_tile_weights":
        (ctypes.c_int, [_c_vp, _c_i64, _c_i64, _c_vp, _c_vp]),
    "fp8w8a8_fp8_linear_group":
        (ctypes.c_int, [_c_vp, ctypes.c_int, _c_i64, _c_vp]),
    "fp8w8a8_group_requant_workspace_bytes":
        (_c_sz, [_c_vp, ctypes.c_int, _c_i64, ctypes.c_int]),
    "fp8w8a8_fp8_linear_group_requant":
        (ctypes.c_int, [_c_vp, ctypes.c_int, _c_i64, ctypes.c_int, _c_vp, _c_vp, _c_vp,
                        _c_sz, _c_vp]),
    "fp8w8a8_rmsnorm_quant_linear":
        (ctypes.c_int, [_c_vp, _c_i64, _c_vp, ctypes.c_float, _c_vp, _c_vp, _c_i64,
                        _c_i64, _c_i64, _c_vp, _c_i64, _c_vp, _c_sz, _c_vp]),
    "fp8w8a8_swiglu_quant_linear":
        (ctypes.c_int, [_c_vp, _c_i64, _c_vp, _c_i64, _c_vp, _c_vp, _c_i64, _c_i64,
                        _c_i64, _c_vp, _c_i64, _c_vp, _c_sz, _c_vp]),
    "fp8w8a8_workspace_bytes": (_c_sz, [_c_i64, _c_i64, _c_i64, ctypes.c_int]),
    "fp8w8a8_workspace_init": (ctypes.c_int, [_c_vp, _c_sz, _c_vp]),
    "fp8w8a8_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "fp8w8a8_last_hip_error": (ctypes.c_int, []),
}

STATUS = {0: "OK", 1: "ERR_NULL", 2: "ERR_SHAPE", 3: "ERR_ALIGN",
          4: "ERR_ALIAS", 5: "ERR_WORKSPACE", 6: "ERR_DEVICE", 7: "ERR_HIP"}

_lib = None
_lib_lock = threading.Lock()


class Fp8W8A8Error(RuntimeError):
    """A non-zero status returned by the library."""

    def __init__(self, status: int, what: str):
        lib = load_library()
        msg = lib.fp8w8a8_status_string(status).decode()
        if status in (6, 7):
            msg += f" (hipError {lib.fp8w8a8_last_hip_error()})"
        super().__init__(f"{what}: {msg}")
        self.status = status


def load_library(path: str = LIBRARY_PATH):
    """Load the HIP library once; raise if it has not been built."""
    global _lib
    with _lib_lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is missing: build it with "
                "`python -m fp8_w8a8_dynamic_amd.build` (no fallback exists)")
        lib = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
        return lib


def _check(status: int, what: str):
    if status != 0:
        raise Fp8W8A8Error(status, what)


def _stream_ptr(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _scales(t: torch.Tensor, count: int, device, name: str) -> torch.Tensor:
    """float32 scales: one per row, contiguous, on the operands' device (the
    kernels read exactly `count` of them)."""
    if not isinstance(t, torch.Tensor) or t.dtype != torch.float32:
        raise TypeError(f"{name} must be a float32 tensor")
    if t.device != device or t.numel() != count or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous float32 tensor of {count} "
                         f"elements on {device}")
    return t


def _as_codes(t: torch.Tensor) -> torch.Tensor:
    """Accept E4M3 tensors as float8_e4m3fn or as raw uint8 bytes."""
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8)
    if t.dtype != torch.uint8:
        raise TypeError(f"expected float8_e4m3fn or uint8 codes, got {t.dtype}")
    return t


def _rows(t: torch.Tensor, name: str):
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D tensor with contiguous rows")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    return t.shape[0], t.shape[1], t.stride(0)


class _Workspaces:
    """One scratch workspace per (device, stream), grown on demand (calls on
    one stream are ordered, so they can share it)."""

    def __init__(self):
        self._bufs = {}
        self._lock = threading.Lock()

    def get(self, device: torch.device, nbytes: int) -> torch.Tensor:
        if nbytes == 0:
            return None
        stream = torch.cuda.current_stream(device)
        key = (device.index, stream.cuda_stream)
        with self._lock:
            buf = self._bufs.get(key)
            if buf is None or buf.numel() < nbytes:
                size = max(nbytes, 1 << 20)
                size = (size + 255) // 256 * 256
                buf = torch.empty(size, dtype=torch.uint8, device=device)
                self._bufs[key] = buf
            return buf


_workspaces = _Workspaces()


def workspace_bytes(m: int, n: int, k: int, fused) -> int:
    """Workspace for fp8_linear (fused 0 / False), quant_linear (1 / True),
    rmsnorm_quant_linear (2) or swiglu_quant_linear (3)."""
    return int(load_library().fp8w8a8_workspace_bytes(m, n, k, int(fused)))


def init_workspace(ws: torch.Tensor) -> torch.Tensor:
    """Zero a caller-owned uint8 workspace with the library's fill kernel."""
    if ws.dtype != torch.uint8 or not ws.is_cuda or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 device tensor")
    _check(load_library().fp8w8a8_workspace_init(
        ws.data_ptr(), ws.numel(), _stream_ptr(ws.device)), "workspace_init")
    return ws


def _pick_workspace(device, need, workspace):
    if workspace is None:
        return _workspaces.get(device, need)
    if need and workspace.numel() < need:
        raise ValueError(f"workspace has {workspace.numel()} bytes, needs {need}")
    return workspace


def quantize_weight_channelwise(w: torch.Tensor):
    """bf16 W[N, K] -> (qW float8_e4m3fn [N, K], w_scale float32 [N])."""
    lib = load_library()
    if w.dtype != torch.bfloat16:
        raise TypeError("w must be bfloat16")
    n, k, ld = _rows(w, "w")
    qw = torch.empty((n, k), dtype=torch.uint8, device=w.device)
    sw = torch.empty((n,), dtype=torch.float32, device=w.device)
    if n == 0:
        return qw.view(torch.float8_e4m3fn), sw
    _check(lib.fp8w8a8_quantize_weight_channelwise(
        w.data_ptr(), n, k, ld, qw.data_ptr(), sw.data_ptr(),
        _stream_ptr(w.device)), "quantize_weight_channelwise")
    return qw.view(torch.float8_e4m3fn), sw


def quantize_act_per_token(x: torch.Tensor):
    """bf16 X[M, K] -> (qX float8_e4m3fn [M, K], x_scale float32 [M])."""
    lib = load_library()
    if x.dtype != torch.bfloat16:
        raise TypeError("x must be bfloat16")
    m, k, ld = _rows(x, "x")
    qx = torch.empty((m, k), dtype=torch.uint8, device=x.device)
    sx = torch.empty((m,), dtype=torch.float32, device=x.device)
    if m == 0:
        return qx.view(torch.float8_e4m3fn), sx
    _check(lib.fp8w8a8_quantize_act_per_token(
        x.data_ptr(), m, k, ld, qx.data_ptr(), sx.data_ptr(),
        _stream_ptr(x.device)), "quantize_act_per_token")
    return qx.view(torch.float8_e4m3fn), sx


def rmsnorm_quantize(x: torch.Tensor, gamma: torch.Tensor, eps: float,
                     return_normed: bool = False, out: torch.Tensor = None):
    """BF16 RMSNorm of X[M, K] with weight gamma[K], then the per-token
    quantization of the norm's bf16 output.

    Returns ``(qX float8_e4m3fn [M, K], x_scale float32 [M])``, plus the
    bf16 norm output [M, K] as a third item when ``return_normed`` is set or
    ``out`` (a bf16 [M, K] tensor with contiguous rows) is given."""
    lib = load_library()
    if x.dtype != torch.bfloat16 or gamma.dtype != torch.bfloat16:
        raise TypeError("x and gamma must be bfloat16")
    m, k, ld = _rows(x, "x")
    if (gamma.dim() != 1 or gamma.numel() != k or not gamma.is_contiguous()
            or gamma.device != x.device):
        raise ValueError(f"gamma must be a contiguous bf16 tensor of {k} elements "
                         f"on {x.device}")
    eps = float(eps)
    qx = torch.empty((m, k), dtype=torch.uint8, device=x.device)
    sx = torch.empty((m,), dtype=torch.float32, device=x.device)
    y = None
    if return_normed or out is not None:
        y = _out(m, k, x.device, out)
    if m > 0:
        _check(lib.fp8w8a8_rmsnorm_quantize(
            x.data_ptr(), m, k, ld, gamma.data_ptr(), eps, qx.data_ptr(),
            sx.data_ptr(), y.data_ptr() if y is not None else None,
            y.stride(0) if y is not None else 0, _stream_ptr(x.device)),
            "rmsnorm_quantize")
    if y is None:
        return qx.view(torch.float8_e4m3fn), sx
    return qx.view(torch.float8_e4m3fn), sx, y


def swiglu_quantize(gate: torch.Tensor, up: torch.Tensor,
                    return_h: bool = False, out: torch.Tensor = None):
    """h = bf16(bf16(silu(gate)) * up) over [M, N], then the per-token
    quantization of h (the input of down_proj).  gate and up may be strided
    views, e.g. the two halves of gate_up_proj's output.

    Returns ``(qH float8_e4m3fn [M, N], h_scale float32 [M])``, plus h (bf16
    [M, N]) as a third item when ``return_h`` is set or ``out`` is given."""
    lib = load_library()
    if gate.dtype != torch.bfloat16 or up.dtype != torch.bfloat16:
        raise TypeError("gate and up must be bfloat16")
    m, n, ldg = _rows(gate, "gate")
    m2, n2, ldu = _rows(up, "up")
    if (m2, n2) != (m, n) or up.device != gate.device:
        raise ValueError("gate and up must have one shape and one device")
    qh = torch.empty((m, n), dtype=torch.uint8, device=gate.device)
    sh = torch.empty((m,), dtype=torch.float32, device=gate.device)
    h = None
    if return_h or out is not None:
        h = _out(m, n, gate.device, out)
    if m > 0:
        _check(lib.fp8w8a8_swiglu_quantize(
            gate.data_ptr(), ldg, up.data_ptr(), ldu, m, n, qh.data_ptr(),
            sh.data_ptr(), h.data_ptr() if h is not None else None,
            h.stride(0) if h is not None else 0, _stream_ptr(gate.device)),
            "swiglu_quantize")
    if h is None:
        return qh.view(torch.float8_e4m3fn), sh
    return qh.view(torch.float8_e4m3fn), sh, h


def kv_quantize_fp8(kv: torch.Tensor, group: int = 128, codes: torch.Tensor = None,
                    scales: torch.Tensor = None):
    """K or V rows [T, W] (bf16, W = kv_heads * head_dim) -> (codes
    float8_e4m3fn [T, W], scales float32 [T, W // group]).  ``codes`` and
    ``scales`` may be given (e.g. slices of a cache's tail: contiguous
    [T, W] / [T, W // group] views)."""
    lib = load_library()
    if kv.dtype != torch.bfloat16:
        raise TypeError("kv must be bfloat16")
    t, w, ld = _rows(kv, "kv")
    if group <= 0 or w % group != 0:
        raise ValueError("the row width must be a multiple of the group")
    codes = torch.empty((t, w), dtype=torch.uint8, device=kv.device) if codes is None \
        else _as_codes(codes)
    scales = torch.empty((t, w // group), dtype=torch.float32, device=kv.device) \
        if scales is None else scales
    if (tuple(codes.shape) != (t, w) or not codes.is_contiguous()
            or codes.device != kv.device):
        raise ValueError(f"codes must be a contiguous [{t}, {w}] tensor on {kv.device}")
    if (scales.dtype != torch.float32 or tuple(scales.shape) != (t, w // group)
            or not scales.is_contiguous() or scales.device != kv.device):
        raise ValueError(f"scales must be a contiguous float32 [{t}, {w // group}] tensor")
    if t > 0:
        _check(lib.fp8w8a8_kv_quantize_fp8(
            kv.data_ptr(), t, w, ld, group, codes.data_ptr(), scales.data_ptr(),
            _stream_ptr(kv.device)), "kv_quantize_fp8")
    return codes.view(torch.float8_e4m3fn), scales


def kv_dequantize_fp8(codes: torch.Tensor, scales: torch.Tensor, group: int = 128,
                      out: torch.Tensor = None):
    """(codes [T, W], scales [T, W // group]) -> bf16 [T, W] =
    bf16(dec(code) * scale)."""
    lib = load_library()
    codes = _as_codes(codes)
    t, w, ldc = _rows(codes, "codes")
    if ldc != w:
        raise ValueError("codes must be contiguous")
    if group <= 0 or w % group != 0:
        raise ValueError("the row width must be a multiple of the group")
    scales = _scales(scales.reshape(-1) if scales.is_contiguous() else scales,
                     t * (w // group), codes.device, "scales")
    y = _out(t, w, codes.device, out)
    if t > 0:
        _check(lib.fp8w8a8_kv_dequantize_fp8(
            codes.data_ptr(), scales.data_ptr(), t, w, group, y.data_ptr(),
            y.stride(0), _stream_ptr(codes.device)), "kv_dequantize_fp8")
    return y


def _group_params(t, count, device, name, given):
    if given is None:
        return torch.empty((t, count), dtype=torch.float32, device=device)
    if (given.dtype != torch.float32 or tuple(given.shape) != (t, count)
            or not given.is_contiguous() or given.device != device):
        raise ValueError(f"{name} must be a contiguous float32 [{t}, {count}] tensor")
    return given


def kv_quantize_int8(kv: torch.Tensor, group: int = 64, codes: torch.Tensor = None,
                     scales: torch.Tensor = None, mins: torch.Tensor = None):
    """K or V rows [T, W] (bf16) -> (codes uint8 [T, W], scales float32
    [T, W // group], mins float32 [T, W // group]), asymmetric min-max per
    group.  Outputs may be given (e.g. the next rows of a cache's INT8
    store)."""
    lib = load_library()
    if kv.dtype != torch.bfloat16:
        raise TypeError("kv must be bfloat16")
    t, w, ld = _rows(kv, "kv")
    if group <= 0 or w % group != 0:
        raise ValueError("the row width must be a multiple of the group")
    codes = torch.empty((t, w), dtype=torch.uint8, device=kv.device) if codes is None \
        else codes
    if (codes.dtype != torch.uint8 or tuple(codes.shape) != (t, w)
            or not codes.is_contiguous() or codes.device != kv.device):
        raise ValueError(f"codes must be a contiguous uint8 [{t}, {w}] tensor")
    scales = _group_params(t, w // group, kv.device, "scales", scales)
    mins = _group_params(t, w // group, kv.device, "mins", mins)
    if t > 0:
        _check(lib.fp8w8a8_kv_quantize_int8(
            kv.data_ptr(), t, w, ld, group, codes.data_ptr(), scales.data_ptr(),
            mins.data_ptr(), _stream_ptr(kv.device)), "kv_quantize_int8")
    return codes, scales, mins


def kv_read_int8(codes: torch.Tensor, scales: torch.Tensor, mins: torch.Tensor,
                 tail: torch.Tensor = None, group: int = 64, out: torch.Tensor = None):
    """The cache read: the dequantized INT8 history [H, W] followed by the
    bf16 residual rows ``tail`` [R, W] -> bf16 [H + R, W]."""
    lib = load_library()
    if codes.dtype != torch.uint8:
        raise TypeError("codes must be uint8")
    h, w, ldc = _rows(codes, "codes")
    if ldc != w:
        raise ValueError("codes must be contiguous")
    if group <= 0 or w % group != 0:
        raise ValueError("the row width must be a multiple of the group")
    scales = _group_params(h, w // group, codes.device, "scales", scales)
    mins = _group_params(h, w // group, codes.device, "mins", mins)
    r, ldt = 0, w
    if tail is not None:
        if tail.dtype != torch.bfloat16:
            raise TypeError("tail must be bfloat16")
        r, w2, ldt = _rows(tail, "tail")
        if w2 != w or tail.device != codes.device:
            raise ValueError("tail must have the history's width and device")
    y = _out(h + r, w, codes.device, out)
    if h + r > 0:
        _check(lib.fp8w8a8_kv_read_int8(
            codes.data_ptr() if h else None, scales.data_ptr() if h else None,
            mins.data_ptr() if h else None, h,
            tail.data_ptr() if r else None, r, ldt, w, group, y.data_ptr(),
            y.stride(0), _stream_ptr(codes.device)), "kv_read_int8")
    return y


def _out(m, n, device, out):
    if out is None:
        return torch.empty((m, n), dtype=torch.bfloat16, device=device)
    if (out.dtype != torch.bfloat16 or tuple(out.shape) != (m, n) or out.stride(1) != 1
            or out.device != device):
        raise ValueError("out must be bfloat16 [M, N] with contiguous rows, on the "
                         "operands' device")
    return out


def fp8_linear(qx, x_scale, qw, w_scale, out=None, workspace=None):
    """Y[M, N] = bf16((qX @ qW^T) * x_scale[:, None] * w_scale[None, :]).

    ``workspace``: optional caller-owned buffer (see :func:`init_workspace`);
    by default a cached per-stream workspace is used."""
    lib = load_library()
    qx, qw = _as_codes(qx), _as_codes(qw)
    m, k, ldq = _rows(qx, "qx")
    n, k2, ldw = _rows(qw, "qw")
    if k2 != k or ldq != k or ldw != k:
        raise ValueError("qx [M, K] and qw [N, K] must be contiguous with one K")
    if qw.device != qx.device:
        raise ValueError("qx and qw must be on one device")
    x_scale = _scales(x_scale, m, qx.device, "x_scale")
    w_scale = _scales(w_scale, n, qx.device, "w_scale")
    y = _out(m, n, qx.device, out)
    if m == 0 or n == 0:
        return y
    need = workspace_bytes(m, n, k, False)
    ws = _pick_workspace(qx.device, need, workspace)
    _check(lib.fp8w8a8_fp8_linear(
        qx.data_ptr(), x_scale.data_ptr(), qw.data_ptr(), w_scale.data_ptr(),
        m, n, k, y.data_ptr(), y.stride(0),
        ws.data_ptr() if ws is not None else None,
        ws.numel() if ws is not None else 0, _stream_ptr(qx.device)),
        "fp8_linear")
    return y


def fp8_linear_requant(qx, x_scale, qw, w_scale, out=None, workspace=None):
    """:func:`fp8_linear` whose output is also quantized per token for the
    Linear that reads it next.

    Returns ``(y bf16 [M, N], qy float8_e4m3fn [M, N], y_scale float32 [M])``:
    y as :func:`fp8_linear` gives it and ``(qy, y_scale)`` as
    :func:`quantize_act_per_token` gives them for y."""
    lib = load_library()
    qx, qw = _as_codes(qx), _as_codes(qw)
    m, k, ldq = _rows(qx, "qx")
    n, k2, ldw = _rows(qw, "qw")
    if k2 != k or ldq != k or ldw != k:
        raise ValueError("qx [M, K] and qw [N, K] must be contiguous with one K")
    if qw.device != qx.device:
        raise ValueError("qx and qw must be on one device")
    x_scale = _scales(x_scale, m, qx.device, "x_scale")
    w_scale = _scales(w_scale, n, qx.device, "w_scale")
    y = _out(m, n, qx.device, out)
    qy = torch.empty((m, n), dtype=torch.uint8, device=qx.device)
    sy = torch.empty((m,), dtype=torch.float32, device=qx.device)
    if m == 0 or n == 0:
        return y, qy.view(torch.float8_e4m3fn), sy
    need = workspace_bytes(m, n, k, False)
    ws = _pick_workspace(qx.device, need, workspace)
    _check(lib.fp8w8a8_fp8_linear_requant(
        qx.data_ptr(), x_scale.data_ptr(), qw.data_ptr(), w_scale.data_ptr(),
        m, n, k, y.data_ptr(), y.stride(0), qy.data_ptr(), sy.data_ptr(),
        ws.data_ptr() if ws is not None else None,
        ws.numel() if ws is not None else 0, _stream_ptr(qx.device)),
        "fp8_linear_requant")
    return y, qy.view(torch.float8_e4m3fn), sy


def quant_linear(x, qw, w_scale, out=None, workspace=None):
    """Fused FP8_DYNAMIC forward: bf16 X[M, K] -> bf16 Y[M, N]."""
    lib = load_library()
    if x.dtype != torch.bfloat16:
        raise TypeError("x must be bfloat16")
    qw = _as_codes(qw)
    m, k, ldx = _rows(x, "x")
    n, k2, ldw = _rows(qw, "qw")
    if k2 != k or ldw != k:
        raise ValueError("qw must be contiguous [N, K] with the K of x")
    if qw.device != x.device:
        raise ValueError("x and qw must be on one device")
    w_scale = _scales(w_scale, n, x.device, "w_scale")
    y = _out(m, n, x.device, out)
    if m == 0 or n == 0:
        return y
    need = workspace_bytes(m, n, k, True)
    ws = _pick_workspace(x.device, need, workspace)
    _check(lib.fp8w8a8_quant_linear(
        x.data_ptr(), ldx, qw.data_ptr(), w_scale.data_ptr(), m, n, k,
        y.data_ptr(), y.stride(0), ws.data_ptr() if ws is not None else None,
        ws.numel() if ws is not None else 0, _stream_ptr(x.device)),
        "quant_linear")
    return y


def quant_linear_noalloc(x, qw, w_scale, out=None):
    """The fused forward without a workspace: the library stages what it
    needs in its own per-GPU scratch array (no allocation by the library;
    calls that overlap on one GPU race).  Same results as quant_linear."""
    lib = load_library()
    if x.dtype != torch.bfloat16:
        raise TypeError("x must be bfloat16")
    qw = _as_codes(qw)
    m, k, ldx = _rows(x, "x")
    n, k2, ldw = _rows(qw, "qw")
    if k2 != k or ldw != k:
        raise ValueError("qw must be contiguous [N, K] with the K of x")
    if qw.device != x.device:
        raise ValueError("x and qw must be on one device")
    w_scale = _scales(w_scale, n, x.device, "w_scale")
    y = _out(m, n, x.device, out)
    if m == 0 or n == 0:
        return y
    _check(lib.fp8w8a8_quant_linear_noalloc(
        x.data_ptr(), ldx, qw.data_ptr(), w_scale.data_ptr(), m, n, k,
        y.data_ptr(), y.stride(0), _stream_ptr(x.device)), "quant_linear_noalloc")
    return y


class _GroupLinear(ctypes.Structure):
    """Mirror of fp8w8a8_group_linear."""
    _fields_ = [("x", _c_vp), ("qw", _c_vp), ("w_scale", _c_vp), ("y", _c_vp),
                ("n", _c_i64), ("k", _c_i64)]


def quant_linear_group_m1(xs, qws, w_scales, outs=None):
    """Several independent one-token FP8_DYNAMIC forwards in one launch:
    xs[i] bf16 [1, K_i] -> outs[i] bf16 [1, N_i], each bit-identical to
    quant_linear(xs[i], qws[i], w_scales[i])."""
    lib = load_library()
    count = len(xs)
    if not (len(qws) == len(w_scales) == count) or (outs is not None and len(outs) != count):
        raise ValueError("one qw, w_scale (and out) per x")
    items = (_GroupLinear * max(count, 1))()
    ys = []
    for i, (x, qw, sw) in enumerate(zip(xs, qws, w_scales)):
        if x.dtype != torch.bfloat16:
            raise TypeError("x must be bfloat16")
        qw = _as_codes(qw)
        m, k, _ = _rows(x, "x")
        n, k2, ldw = _rows(qw, "qw")
        if m != 1 or k2 != k or ldw != k or qw.device != x.device:
            raise ValueError("each x must be [1, K] with qw [N, K] contiguous on its device")
        sw = _scales(sw, n, x.device, "w_scale")
        y = _out(1, n, x.device, None if outs is None else outs[i])
        if not y.is_contiguous():
            raise ValueError("each out must be contiguous")
        items[i] = _GroupLinear(x.data_ptr(), qw.data_ptr(), sw.data_ptr(), y.data_ptr(),
                                n, k)
        ys.append(y)
    if count == 0:
        return ys
    _check(lib.fp8w8a8_quant_linear_group_m1(items, count, _stream_ptr(xs[0].device)),
           "quant_linear_group_m1")
    return ys


class _GroupQuant(ctypes.Structure):
    """Mirror of fp8w8a8_group_quant."""
    _fields_ = [("x", _c_vp), ("m", _c_i64), ("k", _c_i64), ("ldx", _c_i64),
                ("qx", _c_vp), ("x_scale", _c_vp)]


def quantize_act_group(xs):
    """Per-token quantization of several bf16 matrices in one launch:
    [(qX float8_e4m3fn [M_i, K_i], x_scale float32 [M_i]) for each X_i],
    each bit-identical to quantize_act_per_token(X_i)."""
    lib = load_library()
    count = len(xs)
    items = (_GroupQuant * max(count, 1))()
    outs = []
    for i, x in enumerate(xs):
        if x.dtype != torch.bfloat16:
            raise TypeError("each x must be bfloat16")
        m, k, ld = _rows(x, "x")
        if x.device != xs[0].device:
            raise ValueError("every x must be on one device")
        qx = torch.empty((m, k), dtype=torch.uint8, device=x.device)
        sx = torch.empty((m,), dtype=torch.float32, device=x.device)
        items[i] = _GroupQuant(x.data_ptr(), m, k, ld, qx.data_ptr(), sx.data_ptr())
        outs.append((qx.view(torch.float8_e4m3fn), sx))
    if count == 0:
        return outs
    _check(lib.fp8w8a8_quantize_act_group(items, count, _stream_ptr(xs[0].device)),
           "quantize_act_group")
    return outs


def tile_weights(qw, out=None):
    """E4M3 weight codes [N, K] (row-major, as quantized) -> the same bytes
    in MFMA-tile order (uint8, N * K), the weight layout of
    fp8_linear_group."""
    lib = load_library()
    qw = _as_codes(qw)
    n, k, ldw = _rows(qw, "qw")
    if ldw != k:
        raise ValueError("qw must be contiguous [N, K]")
    if out is None:
        out = torch.empty((n * k,), dtype=torch.uint8, device=qw.device)
    elif (out.dtype != torch.uint8 or out.numel() != n * k or not out.is_contiguous()
          or out.device != qw.device):
        raise ValueError(f"out must be a contiguous uint8 tensor of {n * k} bytes on {qw.device}")
    _check(lib.fp8w8a8_tile_weights(qw.data_ptr(), n, k, out.data_ptr(),
                                    _stream_ptr(qw.device)), "tile_weights")
    return out


class _GroupFp8Linear(ctypes.Structure):
    """Mirror of fp8w8a8_group_fp8_linear."""
    _fields_ = [("qx", _c_vp), ("x_scale", _c_vp), ("qw_tiled", _c_vp), ("w_scale", _c_vp),
                ("y", _c_vp), ("n", _c_i64), ("k", _c_i64)]


def _group_items(qxs, x_scales, qws_tiled, w_scales, ns, outs):
    """The items array of a grouped call on given codes, with the outputs."""
    count = len(qxs)
    if (not (len(x_scales) == len(qws_tiled) == len(w_scales) == len(ns) == count)
            or (outs is not None and len(outs) != count)):
        raise ValueError("one x_scale, tiled qw, w_scale, n (and out) per qx")
    items = (_GroupFp8Linear * max(count, 1))()
    ys, m0 = [], None
    for i, (qx, sx, qt, sw, n) in enumerate(zip(qxs, x_scales, qws_tiled, w_scales, ns)):
        qx = _as_codes(qx)
        m, k, ldq = _rows(qx, "qx")
        if ldq != k:
            raise ValueError("each qx must be contiguous [M, K]")
        if m0 is None:
            m0 = m
        elif m != m0 or qx.device != qxs[0].device:
            raise ValueError("every qx must have the same M, on one device")
        if (qt.dtype != torch.uint8 or qt.numel() != n * k or not qt.is_contiguous()
                or qt.device != qx.device):
            raise ValueError(f"tiled weights must be contiguous uint8, {n} x {k} bytes, "
                             "on the codes' device")
        sx = _scales(sx, m, qx.device, "x_scale")
        sw = _scales(sw, n, qx.device, "w_scale")
        y = _out(m, n, qx.device, None if outs is None else outs[i])
        if not y.is_contiguous():
            raise ValueError("each out must be contiguous")
        items[i] = _GroupFp8Linear(qx.data_ptr(), sx.data_ptr(), qt.data_ptr(),
                                   sw.data_ptr(), y.data_ptr(), n, k)
        ys.append(y)
    return items, ys, m0


def fp8_linear_group(qxs, x_scales, qws_tiled, w_scales, ns, outs=None):
    """Several Linears on given codes at one token count M (1..256) in one
    launch: outs[i] bf16 [M, ns[i]] = fp8_linear(qxs[i], x_scales[i], W_i,
    w_scales[i]) up to float32 summation order, with qws_tiled[i] =
    tile_weights(W_i).  Items may share qx and x_scale (pass the same
    tensors)."""
    lib = load_library()
    items, ys, m0 = _group_items(qxs, x_scales, qws_tiled, w_scales, ns, outs)
    if not ys:
        return ys
    _check(lib.fp8w8a8_fp8_linear_group(items, len(ys), m0, _stream_ptr(qxs[0].device)),
           "fp8_linear_group")
    return ys


def fp8_linear_group_requant(qxs, x_scales, qws_tiled, w_scales, ns, rq, outs=None,
                             workspace=None, requant=True):
    """fp8_linear_group whose item rq has its K summed in ranges spread over
    the launch, then added in order, and (requant=True) its output quantized
    per token: returns (ys, qy float8_e4m3fn [M, ns[rq]], y_scale float32
    [M]) with (qy, y_scale) = quantize_act_per_token(ys[rq]), or (ys, None,
    None) with requant=False."""
    lib = load_library()
    items, ys, m0 = _group_items(qxs, x_scales, qws_tiled, w_scales, ns, outs)
    if not ys:
        raise ValueError("at least one item")
    count = len(ys)
    if not 0 <= rq < count:
        raise ValueError(f"rq must index one of the {count} items")
    dev = ys[0].device
    qy = torch.empty((m0, ns[rq]), dtype=torch.uint8, device=dev) if requant else None
    sy = torch.empty((m0,), dtype=torch.float32, device=dev) if requant else None
    need = int(lib.fp8w8a8_group_requant_workspace_bytes(items, count, m0, rq))
    ws = _pick_workspace(dev, need, workspace)
    _check(lib.fp8w8a8_fp8_linear_group_requant(
        items, count, m0, rq, qy.data_ptr() if requant else None,
        sy.data_ptr() if requant else None,
        ws.data_ptr() if ws is not None else None, ws.numel() if ws is not None else 0,
        _stream_ptr(dev)), "fp8_linear_group_requant")
    if not requant:
        return ys, None, None
    return ys, qy.view(torch.float8_e4m3fn), sy


def rmsnorm_quant_linear(x, gamma, eps, qw, w_scale, out=None, workspace=None):
    """RMSNorm of x [M, K] with weight gamma [K], then the FP8_DYNAMIC
    Linear: bit-identical to fp8_linear(*rmsnorm_quantize(x, gamma, eps),
    qw, w_scale), one kernel at decode sizes."""
    lib = load_library()
    if x.dtype != torch.bfloat16 or gamma.dtype != torch.bfloat16:
        raise TypeError("x and gamma must be bfloat16")
    qw = _as_codes(qw)
    m, k, ldx = _rows(x, "x")
    n, k2, ldw = _rows(qw, "qw")
    if k2 != k or ldw != k or qw.device != x.device:
        raise ValueError("qw must be contiguous [N, K] with the K of x, on x's device")
    if (gamma.dim() != 1 or gamma.numel() != k or not gamma.is_contiguous()
            or gamma.device != x.device):
        raise ValueError(f"gamma must be a contiguous bf16 tensor of {k} elements")
    w_scale = _scales(w_scale, n, x.device, "w_scale")
    y = _out(m, n, x.device, out)
    if m == 0 or n == 0:
        return y
    ws = _pick_workspace(x.device, workspace_bytes(m, n, k, 2), workspace)
    _check(lib.fp8w8a8_rmsnorm_quant_linear(
        x.data_ptr(), ldx, gamma.data_ptr(), float(eps), qw.data_ptr(),
        w_scale.data_ptr(), m, n, k, y.data_ptr(), y.stride(0),
        ws.data_ptr() if ws is not None else None, ws.numel() if ws is not None else 0,
        _stream_ptr(x.device)), "rmsnorm_quant_linear")
    return y


def swiglu_quant_linear(gate, up, qw, w_scale, out=None, workspace=None):
    """h = bf16(bf16(silu(gate)) * up), then the FP8_DYNAMIC Linear:
    bit-identical to fp8_linear(*swiglu_quantize(gate, up), qw, w_scale),
    one kernel at decode sizes."""
    lib = load_library()
    if gate.dtype != torch.bfloat16 or up.dtype != torch.bfloat16:
        raise TypeError("gate and up must be bfloat16")
    qw = _as_codes(qw)
    m, k, ldg = _rows(gate, "gate")
    m2, k3, ldu = _rows(up, "up")
    n, k2, ldw = _rows(qw, "qw")
    if (m2, k3) != (m, k) or k2 != k or ldw != k:
        raise ValueError("gate, up [M, K] and qw [N, K] must agree")
    if up.device != gate.device or qw.device != gate.device:
        raise ValueError("gate, up and qw must be on one device")
    w_scale = _scales(w_scale, n, gate.device, "w_scale")
    y = _out(m, n, gate.device, out)
    if m == 0 or n == 0:
        return y
    ws = _pick_workspace(gate.device, workspace_bytes(m, n, k, 3), workspace)
    _check(lib.fp8w8a8_swiglu_quant_linear(
        gate.data_ptr(), ldg, up.data_ptr(), ldu, qw.data_ptr(), w_scale.data_ptr(),
        m, n, k, y.data_ptr(), y.stride(0),
        ws.data_ptr() if ws is not None else None, ws.numel() if ws is not None else 0,
        _stream_ptr(gate.device)), "swiglu_quant_linear")
    return y
