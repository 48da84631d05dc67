"""The allocation-free fused forward, fp8w8a8_quant_linear_noalloc (for
callers that cannot allocate: graph capture, serving loops), against the
fused forward with a caller workspace, fp8w8a8_quant_linear, on identical
inputs: the same kernels run, so the outputs must be bit-identical, and
both within the tolerance of the oracle.  Two calls in a row on the
library's shared per-GPU scratch, the second with a smaller input (a
larger and then a smaller staging footprint, and a different kernel path),
then a call beyond the scratch size, which is refused."""

import numpy as np
import pytest
import torch

import fp8_w8a8_dynamic_amd as fq
import oracle
from oracle import check_bytes, check_close
from tests.gpu_util import host_bits, to_dev_bf16
from workloads import bf16_from_f64
from workloads.generators import weight_bf16

pytestmark = pytest.mark.gpu

# (m, n, k): the first call of each pair is the larger one.
PAIRS = [
    ((4096, 4096, 4096), (300, 1040, 4096)),   # GEMM, codes staged; then split-K
    ((2048, 4096, 12288), (16, 4096, 12288)),  # GEMM at K = 12288; then token GEMV
    ((64, 4096, 4096), (1, 1024, 4096)),       # split-K; then fused M = 1 GEMV
]


def _inputs(m, n, k, seed):
    rng = np.random.default_rng(seed)
    x = bf16_from_f64(rng.standard_normal((m, k)) *
                      np.where(rng.random((m, k)) < 0.01, 20.0, 1.0))
    w = weight_bf16(9, seed, 0, n, k)
    return x, w


def _one(m, n, k, seed):
    x, w = _inputs(m, n, k, seed)
    xd = to_dev_bf16(x)
    qw, sw = fq.quantize_weight_channelwise(to_dev_bf16(w))
    y_na = fq.quant_linear_noalloc(xd, qw, sw)
    y_ws = fq.quant_linear(xd, qw, sw)
    torch.cuda.synchronize()
    a, b = host_bits(y_na), host_bits(y_ws)
    check_bytes(a, b, f"noalloc vs workspace {m}x{n}x{k}")
    rows = np.sort(np.random.default_rng(seed).choice(m, min(m, 256), replace=False))
    rq, rs = oracle.quant_act_ref(x[rows])
    y64 = oracle.linear_ref(rq, rs, host_bits(qw), host_bits(sw))
    check_close(a[rows], y64, f"noalloc vs oracle {m}x{n}x{k}")


@pytest.mark.parametrize("first,second", PAIRS)
def test_noalloc_matches_workspace_call_twice(first, second):
    _one(*first, seed=first[0] + first[2])
    _one(*second, seed=second[0] + second[2])


def test_noalloc_refuses_oversized_staging():
    m, n, k = 16384, 256, 4096            # 64 MiB + 64 KiB of codes and scales
    x = torch.zeros((m, k), dtype=torch.bfloat16, device="cuda")
    qw = torch.zeros((n, k), dtype=torch.uint8, device="cuda")
    sw = torch.ones(n, dtype=torch.float32, device="cuda")
    with pytest.raises(fq.Fp8W8A8Error) as ei:
        fq.quant_linear_noalloc(x, qw, sw)
    assert ei.value.status == 5                # FP8W8A8_ERR_WORKSPACE
    # and the library is still usable afterwards
    _one(32, 256, 4096, seed=7)
