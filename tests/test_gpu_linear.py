"""GPU parity of the W8A8 Linear (decode GEMV and prefill GEMM paths)
against the oracle: bf16 outputs within the elementwise tolerance of
oracle.check (1e-2 relative to the oracle's magnitude), quantized bytes
bit-exact.  Calls go through the C ABI via the Python binding."""

import os

import numpy as np
import pytest
import torch

import fp8_w8a8_dynamic_amd as fq
import oracle
from oracle import check_bytes, check_close
from tests.gpu_util import host_bits, to_dev_bf16, to_dev_f32, to_dev_u8
from tests.oracle_par import quant_rows_par
from workloads import LAYER_SHAPES, bf16_from_f64, c1_inputs, c2_inputs, c3_inputs
from workloads.generators import c5_rows, c5_x, weight_bf16

pytestmark = pytest.mark.gpu


def _rand_codes(rng, shape):
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x7E          # no NaN codes
    return c


def _rand_operands(m, n, k, seed):
    rng = np.random.default_rng(seed)
    qx, qw = _rand_codes(rng, (m, k)), _rand_codes(rng, (n, k))
    sx = (2.0 ** rng.uniform(-12, -4, m)).astype(np.float32)
    sw = (2.0 ** rng.uniform(-12, -4, n)).astype(np.float32)
    return qx, sx, qw, sw


def _run_linear(qx, sx, qw, sw):
    y = fq.fp8_linear(to_dev_u8(qx), to_dev_f32(sx), to_dev_u8(qw), to_dev_f32(sw))
    torch.cuda.synchronize()
    return host_bits(y)


SHAPES = [(1, 16, 128), (4, 48, 384), (8, 272, 1024), (16, 1040, 512),
          (17, 16, 128), (100, 272, 384), (300, 1040, 256), (513, 528, 640),
          (256, 256, 4096), (64, 4096, 256), (2, 4096, 4096), (1, 1024, 12288)]


@pytest.mark.parametrize("m,n,k", SHAPES)
def test_fp8_linear_random_codes(m, n, k):
    qx, sx, qw, sw = _rand_operands(m, n, k, m * 1000 + n + k)
    y = _run_linear(qx, sx, qw, sw)
    check_close(y, oracle.linear_ref(qx, sx, qw, sw), f"linear {m}x{n}x{k}")


@pytest.mark.parametrize("m", [1, 4, 8, 16])
@pytest.mark.parametrize("path", ["gemm", "gemv"])
def test_forced_path_cross_check(m, path, monkeypatch):
    """GEMV and GEMM on identical decode-sized inputs, both vs the oracle."""
    monkeypatch.setenv("FP8W8A8_FORCE_PATH", path)
    qx, sx, qw, sw = _rand_operands(m, 1024, 4096, 77 + m)
    y = _run_linear(qx, sx, qw, sw)
    check_close(y, oracle.linear_ref(qx, sx, qw, sw), f"{path} m={m}")


GEMV_CASES = [(1, 48, 384), (2, 16, 640), (3, 272, 4096), (4, 48, 2176),
              (5, 1040, 1024), (8, 48, 256), (9, 64, 12288), (16, 272, 384),
              (1, 1024, 12288), (16, 1024, 4096)]


@pytest.mark.parametrize("gpw", ["1", "2", "3", "7"])
@pytest.mark.parametrize("m,n,k", GEMV_CASES)
def test_every_gemv_grouping(gpw, m, n, k, monkeypatch):
    """Every row-group count per workgroup of the decode kernel (which moves
    the row-group boundaries between its waves, and past 8 items per wave
    switches to batched loads), on ragged token counts and K not a multiple
    of the 2 KB class span, unfused and fused (bf16 in), against the
    oracle."""
    monkeypatch.setenv("FP8W8A8_FORCE_PATH", "gemv")
    monkeypatch.setenv("FP8W8A8_GEMV_GPW", gpw)
    qx, sx, qw, sw = _rand_operands(m, n, k, 31 * m + n + k)
    y = _run_linear(qx, sx, qw, sw)
    check_close(y, oracle.linear_ref(qx, sx, qw, sw), f"gemv gpw {gpw} {m}x{n}x{k}")
    rng = np.random.default_rng(m + k)
    x = bf16_from_f64(rng.standard_normal((m, k)) * 3.0)
    yf = fq.quant_linear(to_dev_bf16(x), to_dev_u8(qw), to_dev_f32(sw))
    torch.cuda.synchronize()
    y64, _, _ = oracle.quant_linear_ref(x, qw, sw)
    check_close(host_bits(yf), y64, f"fused gemv gpw {gpw} {m}x{n}x{k}")


def _quant_weights_gpu(w_bits):
    qw, sw = fq.quantize_weight_channelwise(to_dev_bf16(w_bits))
    return qw, sw


def test_c1_q_proj_end_to_end():
    x, w = c1_inputs()
    qw, sw = _quant_weights_gpu(w)
    y = fq.quant_linear(to_dev_bf16(x), qw, sw)
    torch.cuda.synchronize()
    rqw, rsw = oracle.quant_weight_ref(w)
    check_bytes(host_bits(qw), rqw, "c1 qw")
    check_bytes(host_bits(sw).view(np.uint32), rsw.view(np.uint32), "c1 sw")
    y64, _, _ = oracle.quant_linear_ref(x, rqw, rsw)
    check_close(host_bits(y), y64, "c1 y")


@pytest.mark.parametrize("m", [1, 4, 8])
@pytest.mark.parametrize("linear", range(7))
def test_c2_decode_layer(m, linear):
    x, w = c2_inputs(m, linear)
    qw, sw = _quant_weights_gpu(w)
    y = fq.quant_linear(to_dev_bf16(x), qw, sw)
    torch.cuda.synchronize()
    y64, _, _ = oracle.quant_linear_ref(x, host_bits(qw), host_bits(sw))
    check_close(host_bits(y), y64, f"c2 {LAYER_SHAPES[linear][0]} m={m}")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("linear", range(7))
def test_c3_prefill_all_rows(linear):
    """The 4096-token prefill chunk, each of the 7 Linears in full: weight
    and activation codes and scales bit-exact on every row, every output
    element within the tolerance of the oracle."""
    x, w = c3_inputs(linear, m=4096)
    qw, sw = _quant_weights_gpu(w)
    xd = to_dev_bf16(x)
    y = fq.quant_linear(xd, qw, sw)
    qx, sx = fq.quantize_act_per_token(xd)
    torch.cuda.synchronize()
    name = LAYER_SHAPES[linear][0]
    rq, rs = quant_rows_par(x)
    check_bytes(host_bits(sx).view(np.uint32), rs.view(np.uint32), f"c3 {name} sx")
    check_bytes(host_bits(qx), rq, f"c3 {name} qx")
    rqw, rsw = quant_rows_par(w, weight=True)
    check_bytes(host_bits(sw).view(np.uint32), rsw.view(np.uint32), f"c3 {name} sw")
    check_bytes(host_bits(qw), rqw, f"c3 {name} qw")
    check_close(host_bits(y), oracle.linear_ref(rq, rs, rqw, rsw), f"c3 {name}")


C5_ROWS = 2048


@pytest.mark.timeout(900)
@pytest.mark.parametrize("linear", range(7))
def test_c5_long_prefill(linear):
    """The 16384-token stress chunk (Student-t activations, all-zero rows,
    rows x1e4 and rows saturating E4M3), each of the 7 Linears through the
    fused call: activation codes and scales bit-exact on all 16384 rows
    (K = 4096 and, for down, K = 12288), weight codes on every row, outputs
    on 2048 seeded rows plus every zero and saturating row; zero rows give
    exact zeros."""
    m = 16384
    name, n, k = LAYER_SHAPES[linear]
    x = c5_x(m, k, linear)
    w = weight_bf16(5, 0, linear, n, k)
    qw, sw = _quant_weights_gpu(w)
    xd = to_dev_bf16(x)
    y = fq.quant_linear(xd, qw, sw)
    qx, sx = fq.quantize_act_per_token(xd)
    torch.cuda.synchronize()
    y = host_bits(y)
    rq, rs = quant_rows_par(x)
    check_bytes(host_bits(sx).view(np.uint32), rs.view(np.uint32), f"c5 {name} sx")
    check_bytes(host_bits(qx), rq, f"c5 {name} qx")
    del qx, sx, xd
    rqw, rsw = quant_rows_par(w, weight=True)
    check_bytes(host_bits(sw).view(np.uint32), rsw.view(np.uint32), f"c5 {name} sw")
    check_bytes(host_bits(qw), rqw, f"c5 {name} qw")
    zero, big, heavy = c5_rows(m)
    rows = np.unique(np.concatenate(
        [zero, big, heavy,
         np.random.default_rng(500 + linear).choice(m, C5_ROWS, replace=False)]))
    assert rows.size >= C5_ROWS
    check_close(y[rows], oracle.linear_ref(rq[rows], rs[rows], rqw, rsw), f"c5 {name}")
    assert np.all((y[zero] & 0x7FFF) == 0)


def test_workspace_reuse_across_shapes():
    """One workspace serves calls of different shapes in a row."""
    shapes = [(1, 1024, 4096), (300, 1040, 512), (4, 4096, 12288),
              (1, 1024, 4096), (16, 48, 384), (1, 1024, 4096)]
    for i, (m, n, k) in enumerate(shapes):
        qx, sx, qw, sw = _rand_operands(m, n, k, 500 + i)
        y = _run_linear(qx, sx, qw, sw)
        check_close(y, oracle.linear_ref(qx, sx, qw, sw), f"reuse {i}")


def test_strided_output_and_input():
    rng = np.random.default_rng(12)
    m, n, k = 24, 64, 256
    xfull = bf16_from_f64(rng.standard_normal((m, k + 64)))
    w = bf16_from_f64(rng.standard_normal((n, k)) * 0.02)
    qw, sw = _quant_weights_gpu(w)
    xd = to_dev_bf16(xfull)[:, :k]
    out = torch.zeros((m, n + 40), dtype=torch.bfloat16, device="cuda")
    view = out[:, 8:8 + n]
    fq.quant_linear(xd, qw, sw, out=view)
    torch.cuda.synchronize()
    y64, _, _ = oracle.quant_linear_ref(xfull[:, :k], host_bits(qw), host_bits(sw))
    ob = host_bits(out)
    check_close(ob[:, 8:8 + n], y64, "strided")
    assert np.all(ob[:, :8] == 0) and np.all(ob[:, 8 + n:] == 0)


def test_deterministic_outputs():
    for m in (1, 8, 512):
        qx, sx, qw, sw = _rand_operands(m, 1024, 4096, 900 + m)
        a = _run_linear(qx, sx, qw, sw)
        b = _run_linear(qx, sx, qw, sw)
        assert np.array_equal(a, b)


# (m, n, k, splits): None = the plan's own split (long K), else the 128x64
# configuration forced to that many splits (the plan leaves K <= 4096
# unsplit).
SPLIT_SHAPES = [(17, 4096, 4096, 4), (64, 1024, 4096, 8), (64, 4112, 12288, None),
                (100, 272, 384, 3), (129, 2048, 1152, 5), (256, 4096, 4096, 2),
                (100, 6144, 4096, 2), (48, 4096, 12288, None), (256, 4096, 12288, None)]


@pytest.mark.parametrize("m,n,k,splits", SPLIT_SHAPES)
def test_split_k_gemm(m, n, k, splits, monkeypatch):
    """Token counts with few output tiles split K over workgroups (float32
    partial sums in the workspace, added in split order by a second
    kernel): against the oracle, ragged m and n, uneven splits of K, and
    bit-identical on a second run."""
    monkeypatch.setenv("FP8W8A8_FORCE_PATH", "gemm")
    if splits is not None:
        monkeypatch.setenv("FP8W8A8_GEMM_CONFIG", "5")
        monkeypatch.setenv("FP8W8A8_GEMM_SPLITS", str(splits))
    assert fq.workspace_bytes(m, n, k, False) >= m * n * 4 * 2, "plan does not split K"
    qx, sx, qw, sw = _rand_operands(m, n, k, 7 * m + n + k)
    y = _run_linear(qx, sx, qw, sw)
    check_close(y, oracle.linear_ref(qx, sx, qw, sw), f"split-K {m}x{n}x{k}")
    assert np.array_equal(y, _run_linear(qx, sx, qw, sw))


@pytest.mark.parametrize("m,linear", [(64, 0), (64, 6), (256, 1), (33, 4)])
def test_split_k_fused_layer_shapes(m, linear):
    """The fused call at mid-sized token counts (workspace holding the
    quantized activations and the partial sums) on the layer's shapes."""
    _, n, k = LAYER_SHAPES[linear]
    rng = np.random.default_rng(40 + m + linear)
    x = bf16_from_f64(rng.standard_normal((m, k)))
    w = weight_bf16(2, 0, linear, n, k)
    qw, sw = _quant_weights_gpu(w)
    y = fq.quant_linear(to_dev_bf16(x), qw, sw)
    torch.cuda.synchronize()
    y64, _, _ = oracle.quant_linear_ref(x, host_bits(qw), host_bits(sw))
    check_close(host_bits(y), y64, f"fused split-K m={m} {LAYER_SHAPES[linear][0]}")


TOK_SHAPES = [(17, 16, 128), (31, 272, 384), (32, 1040, 4096), (33, 48, 640),
              (48, 4096, 4096), (63, 1024, 12288), (64, 4112, 1152),
              (64, 4096, 4096)]


@pytest.mark.parametrize("m,n,k", TOK_SHAPES)
def test_token_group_gemv(m, n, k, monkeypatch):
    """16 < m <= 64: the token-group GEMV (2-4 groups of 16 tokens, K split
    over a workgroup's waves, ragged token groups, K ranges of unequal
    length) against the oracle, and bit-identical on a second run."""
    monkeypatch.setenv("FP8W8A8_FORCE_PATH", "tok")
    qx, sx, qw, sw = _rand_operands(m, n, k, 11 * m + n + k)
    y = _run_linear(qx, sx, qw, sw)
    check_close(y, oracle.linear_ref(qx, sx, qw, sw), f"tok {m}x{n}x{k}")
    assert np.array_equal(y, _run_linear(qx, sx, qw, sw))


@pytest.mark.parametrize("m", [17, 40, 64])
@pytest.mark.parametrize("path", ["gemm", "tok"])
def test_token_group_gemv_vs_gemm(m, path, monkeypatch):
    """The token-group GEMV and the (split-K) GEMM on identical inputs, both
    against the oracle."""
    monkeypatch.setenv("FP8W8A8_FORCE_PATH", path)
    qx, sx, qw, sw = _rand_operands(m, 1024, 4096, 300 + m)
    y = _run_linear(qx, sx, qw, sw)
    check_close(y, oracle.linear_ref(qx, sx, qw, sw), f"{path} m={m}")


FINITE_CODES = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)


def _pairs_case(tok_codes, n_codes, k, k0):
    """One-hot operands: token m holds code tok_codes[m] and weight row n
    holds n_codes[n], both at K position k0 and zero elsewhere, unit scales:
    every output is a single E4M3 x E4M3 product, exact in float32, so the
    bf16 output must equal the oracle's bf16 rounding bit for bit."""
    m, n = len(tok_codes), len(n_codes)
    qx = np.zeros((m, k), np.uint8)
    qw = np.zeros((n, k), np.uint8)
    qx[:, k0] = tok_codes
    qw[:, k0] = n_codes
    return qx, np.ones(m, np.float32), qw, np.ones(n, np.float32)


def _check_pairs(qx, sx, qw, sw, what):
    y = _run_linear(qx, sx, qw, sw).copy()
    want = oracle.f64_to_bf16_bits(oracle.linear_ref(qx, sx, qw, sw))
    y[y == 0x8000] = 0                     # a single product of -0 sums to +0
    want = want.copy()
    want[want == 0x8000] = 0
    check_bytes(y, want, what)


@pytest.mark.parametrize("path,cfg", [("gemm", "3"), ("gemm", "4"), ("gemm", "8"),
                                      ("gemm", "10"), ("gemm", "-1"),
                                      ("tok", None)])
def test_all_code_pairs_exact_tiles(path, cfg, monkeypatch):
    """All 254 x 254 finite code pairs through the MFMA tiles (the GEMM's
    configurations, its split-K plan, the token-group GEMV), at K positions
    that reach every 16-byte chunk and both MFMA K halves of a 128-byte
    step."""
    monkeypatch.setenv("FP8W8A8_FORCE_PATH", path)
    if cfg is not None and cfg != "-1":
        monkeypatch.setenv("FP8W8A8_GEMM_CONFIG", cfg)
    codes_n = np.concatenate([FINITE_CODES, np.zeros(2, np.uint8)])   # n = 256
    k = 1024 if cfg == "-1" else 256
    tok_sets = [FINITE_CODES] if path == "gemm" else \
        [FINITE_CODES[i:i + 64] for i in range(0, 254, 64)]
    for k0 in ([0, 17, 63, 64, 100, 127, 128 + 31, 255] + ([700, 1023] if k > 256 else [])):
        for toks in tok_sets:
            qx, sx, qw, sw = _pairs_case(toks, codes_n, k, k0)
            _check_pairs(qx, sx, qw, sw, f"{path} cfg {cfg} k0={k0}")


def test_all_code_pairs_exact_decode_gemv(monkeypatch):
    """All 254 x 254 finite code pairs through the K-class decode GEMV (4
    tokens per call, so four K classes per MFMA), at K positions in every
    class and 16-byte chunk of the first 2 KB."""
    monkeypatch.setenv("FP8W8A8_FORCE_PATH", "gemv")
    codes_n = np.concatenate([FINITE_CODES, np.zeros(2, np.uint8)])
    k = 2048
    for k0 in range(0, 2048, 176):
        for i in range(0, 254, 4):
            qx, sx, qw, sw = _pairs_case(FINITE_CODES[i:i + 4], codes_n, k, k0)
            _check_pairs(qx, sx, qw, sw, f"gemv k0={k0} tokens {i}")


def test_binding_rejects_bad_scales_and_outputs():
    """The binding checks what the kernels would read past: scale dtype,
    length and contiguity, and the output's dtype, shape and device."""
    qx = torch.zeros((4, 128), dtype=torch.uint8, device="cuda")
    qw = torch.zeros((16, 128), dtype=torch.uint8, device="cuda")
    sx = torch.ones(4, dtype=torch.float32, device="cuda")
    sw = torch.ones(16, dtype=torch.float32, device="cuda")
    with pytest.raises(TypeError):
        fq.fp8_linear(qx, sx.to(torch.bfloat16), qw, sw)
    with pytest.raises(ValueError):
        fq.fp8_linear(qx, sx[:3], qw, sw)
    with pytest.raises(ValueError):
        fq.fp8_linear(qx, sx, qw, torch.ones(32, device="cuda")[::2])
    with pytest.raises(ValueError):
        fq.fp8_linear(qx, sx, qw, sw, out=torch.empty((4, 8), dtype=torch.bfloat16, device="cuda"))
    x = torch.zeros((4, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        fq.quant_linear(x, qw, torch.ones(15, device="cuda"))
    y = fq.fp8_linear(qx, sx, qw, sw)
    torch.cuda.synchronize()
    assert y.shape == (4, 16) and not torch.any(y.float() != 0).item()


def test_empty_calls():
    qw = torch.zeros((16, 128), dtype=torch.uint8, device="cuda")
    sw = torch.ones(16, dtype=torch.float32, device="cuda")
    x = torch.zeros((0, 128), dtype=torch.bfloat16, device="cuda")
    y = fq.quant_linear(x, qw, sw)
    assert y.shape == (0, 16)


GEMM_CONFIGS = ["0", "1", "2", "3", "4", "5", "6", "7", "8", "10"]


@pytest.mark.parametrize("m,n,k", [(300, 1040, 384), (513, 528, 640), (4096, 272, 256),
                                   (1, 4096, 128)])
def test_every_gemm_config_matches_oracle_and_each_other(m, n, k, monkeypatch):
    """Every tile configuration accumulates each output over K in the same
    order, so all must agree bit for bit, and with the oracle."""
    qx, sx, qw, sw = _rand_operands(m, n, k, 4242 + m)
    monkeypatch.setenv("FP8W8A8_FORCE_PATH", "gemm")
    y64 = oracle.linear_ref(qx, sx, qw, sw)
    outs = []
    for cfg in GEMM_CONFIGS:
        monkeypatch.setenv("FP8W8A8_GEMM_CONFIG", cfg)
        y = _run_linear(qx, sx, qw, sw)
        check_close(y, y64, f"gemm cfg {cfg} {m}x{n}x{k}")
        outs.append(y)
    for cfg, y in zip(GEMM_CONFIGS[1:], outs[1:]):
        assert np.array_equal(y, outs[0]), f"config {cfg} differs from config 0"


@pytest.mark.parametrize("m", [1, 4, 300])
def test_packed_qkv_equals_separate_calls(m):
    """Packed modules (q|k|v as one Linear with the rows of W and of the
    channel scales concatenated) quantize the shared input once; every
    output channel is the same dot product as in the separate calls, so the
    packed output must match the oracle and, where each output's summation
    order does not depend on N (M = 1 and the tiled GEMM), the separate calls
    bit for bit."""
    rng = np.random.default_rng(7000 + m)
    k = 512
    ws = [bf16_from_f64(rng.standard_normal((n, k)) * 0.02) for n in (256, 64, 64)]
    x = bf16_from_f64(rng.standard_normal((m, k)))
    parts = [_quant_weights_gpu(w) for w in ws]
    qw = torch.cat([p[0].view(torch.uint8) for p in parts])
    sw = torch.cat([p[1] for p in parts])
    xd = to_dev_bf16(x)
    yp = host_bits(fq.quant_linear(xd, qw, sw))
    ys = [host_bits(fq.quant_linear(xd, p[0], p[1])) for p in parts]
    torch.cuda.synchronize()
    y64, _, _ = oracle.quant_linear_ref(x, host_bits(qw), host_bits(sw))
    check_close(yp, y64, f"packed qkv m={m}")
    if m != 4:
        assert np.array_equal(yp, np.concatenate(ys, axis=1))


@pytest.mark.parametrize("n,k", [(4096, 4096), (1024, 4096), (12288, 4096), (4096, 12288),
                                 (6144, 4096), (24576, 4096), (16, 128), (48, 4224),
                                 (1040, 2176), (512, 16384), (8208, 6272)])
@pytest.mark.parametrize("rows", [None, "1", "2", "4"])
def test_m1_kernel_matches_lds_staged_kernel(n, k, rows, monkeypatch):
    """The barrier-free M = 1 GEMV against the LDS-staged one: bitwise where
    the latter gives every wave whole rows (all these shapes), and both
    within the Linear's bound of the oracle."""
    if rows is not None:
        # ignored where steps x rows would exceed 8 items of 2 KB per wave
        monkeypatch.setenv("FP8W8A8_GEMV_M1_ROWS", rows)
    rng = np.random.default_rng(n * 7 + k)
    x = bf16_from_f64(rng.standard_normal((1, k)) * np.where(rng.random(k) < 0.01, 20, 1))
    w = bf16_from_f64(0.02 * rng.standard_normal((n, k)))
    qw, sw = _quant_weights_gpu(w)
    xd = to_dev_bf16(x)
    qx, sx = fq.quantize_act_per_token(xd)
    monkeypatch.setenv("FP8W8A8_GEMV_M1", "1")        # also where K > 4096
    y_new = host_bits(fq.quant_linear(xd, qw, sw))
    c_new = host_bits(fq.fp8_linear(qx, sx, qw, sw))   # codes given
    monkeypatch.setenv("FP8W8A8_GEMV_M1", "0")
    y_old = host_bits(fq.quant_linear(xd, qw, sw))
    c_old = host_bits(fq.fp8_linear(qx, sx, qw, sw))
    torch.cuda.synchronize()
    check_bytes(y_new, y_old, f"m1 kernel vs LDS-staged, n={n} k={k}")
    check_bytes(c_new, c_old, f"m1 kernel on codes vs LDS-staged, n={n} k={k}")
    check_bytes(c_new, y_new, f"m1 kernel on codes vs fused, n={n} k={k}")
    rqx, rsx = oracle.quant_act_ref(x)
    rqw, rsw = oracle.quant_weight_ref(w)
    check_close(y_new, oracle.linear_ref(rqx, rsx, rqw, rsw), f"m1 kernel vs oracle n={n} k={k}")


# fp8w8a8_fp8_linear_requant: K-split shapes, where one kernel adds the
# splits, writes y and quantizes it (n up to 16384), and shapes on the other
# paths (GEMV, token-group GEMV, unsplit GEMM: the Linear, then the
# quantizer).  Each has a zero row (scale 0, codes 0).
REQUANT = [(64, 4096, 12288), (256, 4096, 12288), (64, 1024, 4096), (100, 1040, 1152),
           (1, 1024, 4096), (17, 640, 1024), (4096, 512, 256)]


def _check_requant(m, n, k, seed, what):
    qx, sx, qw, sw = _rand_operands(m, n, k, seed)
    if m > 3:
        qx[3] = 0
    dev = (to_dev_u8(qx), to_dev_f32(sx), to_dev_u8(qw), to_dev_f32(sw))
    y, qy, sy = fq.fp8_linear_requant(*dev)
    y2 = fq.fp8_linear(*dev)
    q2, s2 = fq.quantize_act_per_token(y2)
    torch.cuda.synchronize()
    yb = host_bits(y)
    check_bytes(yb, host_bits(y2), f"{what}: y against fp8_linear")
    check_bytes(host_bits(qy), host_bits(q2), f"{what}: codes against the quantizer on y")
    check_bytes(host_bits(sy).view(np.uint32), host_bits(s2).view(np.uint32),
                f"{what}: scales against the quantizer on y")
    rq, rs = oracle.quant_act_ref(yb)
    check_bytes(host_bits(qy), rq, f"{what}: codes against the oracle")
    check_bytes(host_bits(sy).view(np.uint32), rs.view(np.uint32),
                f"{what}: scales against the oracle")
    check_close(yb, oracle.linear_ref(qx, sx, qw, sw), f"{what}: y against the oracle")


@pytest.mark.parametrize("m,n,k", REQUANT)
def test_fp8_linear_requant(m, n, k):
    _check_requant(m, n, k, 5 * m + n + k, f"requant {m}x{n}x{k}")


@pytest.mark.parametrize("m,n,k,splits", [(64, 2048, 4096, 8), (33, 16384, 1024, 3),
                                          (130, 656, 2048, 5)])
def test_fp8_linear_requant_forced_splits(m, n, k, splits, monkeypatch):
    """More K splits than the planner picks (the 128x64 configuration),
    the longest row the fused kernel takes (n = 16384) and a ragged one."""
    monkeypatch.setenv("FP8W8A8_GEMM_CONFIG", "5")
    monkeypatch.setenv("FP8W8A8_GEMM_SPLITS", str(splits))
    _check_requant(m, n, k, 11 * m + n + splits, f"requant {m}x{n}x{k} {splits} splits")
