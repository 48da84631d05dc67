"""The benchmark's measured-peak kernels run and produce live results: the
MFMA-only loop's accumulators are finite and its clock counters advance;
the streaming read's per-thread XOR reflects the bytes read (a zero buffer
gives zeros, a buffer with one changed word changes exactly one thread's
value)."""

import ctypes

import pytest
import torch

from fp8_w8a8_dynamic_amd import build as fbuild

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def plib():
    lib = ctypes.CDLL(fbuild.PEAKS_LIB_PATH)
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    lib.fp8w8a8_peaks_mfma_out_floats.restype = i64
    lib.fp8w8a8_peaks_mfma_out_floats.argtypes = [i64]
    lib.fp8w8a8_peaks_mfma_loop.argtypes = [vp, vp, i64, ctypes.c_int, vp]
    lib.fp8w8a8_peaks_read_workgroups.restype = i64
    lib.fp8w8a8_peaks_read_workgroups.argtypes = [i64]
    lib.fp8w8a8_peaks_read_stream.argtypes = [vp, i64, vp, vp]
    return lib


def test_mfma_loop_runs(plib):
    wg = 8
    out = torch.full((plib.fp8w8a8_peaks_mfma_out_floats(wg),), float("nan"), device="cuda")
    clk = torch.zeros(2, dtype=torch.int64, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    assert plib.fp8w8a8_peaks_mfma_loop(out.data_ptr(), clk.data_ptr(), wg, 16, st) == 0
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and (out > 0).all()
    cycles, ticks = (int(v) for v in clk.cpu())
    assert cycles > 0 and ticks >= 0


def test_read_stream_reads_every_byte(plib):
    nbytes = 4 << 20
    buf = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    out = torch.full((plib.fp8w8a8_peaks_read_workgroups(nbytes) * 256,), -1,
                     dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    assert plib.fp8w8a8_peaks_read_stream(buf.data_ptr(), nbytes, out.data_ptr(), st) == 0
    torch.cuda.synchronize()
    assert (out == 0).all()
    buf.view(torch.int32)[12345] = 0x5A5A5A5A
    assert plib.fp8w8a8_peaks_read_stream(buf.data_ptr(), nbytes, out.data_ptr(), st) == 0
    torch.cuda.synchronize()
    nz = torch.nonzero(out).flatten()
    assert nz.numel() == 1 and int(out[nz[0]]) == 0x5A5A5A5A
