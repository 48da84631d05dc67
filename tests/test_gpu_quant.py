"""GPU parity of the quantization kernels against the oracle: codes and
float32 scales must be bit-identical.  Calls go through the C ABI via the
Python binding."""

import numpy as np
import pytest
import torch

import fp8_w8a8_dynamic_amd as fq
import oracle
from oracle import check_bytes
from tests.gpu_util import host_bits, to_dev_bf16
from tests.oracle_par import quant_rows_par
from workloads import LAYER_SHAPES, bf16_from_f64, c1_inputs, c2_inputs, c3_inputs
from workloads.generators import c5_rows, c5_x

pytestmark = pytest.mark.gpu


def _gpu_quant(bits, weight=False):
    x = to_dev_bf16(bits)
    if weight:
        q, s = fq.quantize_weight_channelwise(x)
    else:
        q, s = fq.quantize_act_per_token(x)
    torch.cuda.synchronize()
    return host_bits(q), host_bits(s)


def _check_rows(bits, q, s, rows=None, what="quant"):
    ref = bits if rows is None else bits[rows]
    rq, rs = oracle.quant_act_ref(ref)
    gq = q if rows is None else q[rows]
    gs = s if rows is None else s[rows]
    check_bytes(gs.view(np.uint32), rs.view(np.uint32), what + " scales")
    check_bytes(gq, rq, what + " codes")


def _all_finite_bf16():
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    exp = (b >> 7) & 0xFF
    return b[exp != 0xFF]


def test_every_bf16_value_under_many_scales():
    """Each row holds every finite bf16 value whose magnitude is at most the
    row's amax (larger ones replaced by +0) and the amax itself, so every
    bf16 input meets the encoder under each row's scale."""
    allb = _all_finite_bf16()
    mag = oracle.bf16_bits_to_f32(allb & np.uint16(0x7FFF))
    rng = np.random.default_rng(17)
    amaxes = [448.0, 1.0, 896.0, 3.0, 1e-3, 2.0 ** -130, 7.0 * 2.0 ** -133,
              1e30, 0.1, 3.3e38]
    # Scales at the edges of the kernels' hoisted-reciprocal range
    # [2^-60, 2^60] and one bf16 step either side.
    for e in (-60, 60):
        for f in (1.0 - 2.0 ** -7, 1.0, 1.0 + 2.0 ** -6):
            amaxes.append(448.0 * 2.0 ** e * f)
    amaxes += list(2.0 ** rng.uniform(-120, 120, 40))
    amax_bits = bf16_from_f64(np.array(amaxes))
    k = ((allb.size + 1 + 7) // 8) * 8
    rows = np.zeros((len(amaxes), k), np.uint16)
    for r, ab in enumerate(amax_bits):
        amax = oracle.bf16_bits_to_f32(np.array([ab]))[0]
        keep = np.where(mag <= amax, allb, np.uint16(0))
        rows[r, 0] = ab
        rows[r, 1:1 + keep.size] = keep
    q, s = _gpu_quant(rows)
    _check_rows(rows, q, s, what="all-bf16")


def test_c1_activations_and_weights():
    x, w = c1_inputs()
    q, s = _gpu_quant(x)
    _check_rows(x, q, s, what="c1 x")
    qw, sw = _gpu_quant(w, weight=True)
    rq, rs = oracle.quant_weight_ref(w)
    check_bytes(sw.view(np.uint32), rs.view(np.uint32), "c1 w scales")
    check_bytes(qw, rq, "c1 w codes")


@pytest.mark.parametrize("linear", range(7))
def test_c2_weights_sampled_rows(linear):
    _, w = c2_inputs(1, linear)
    qw, sw = _gpu_quant(w, weight=True)
    rows = np.random.default_rng(linear).choice(w.shape[0], 256, replace=False)
    _check_rows(w, qw, sw, rows, what=f"w {LAYER_SHAPES[linear][0]}")


@pytest.mark.timeout(300)
@pytest.mark.parametrize("linear", [0, 6])
def test_c3_activations(linear):
    """Codes and scales of the prefill chunk's K = 4096 and K = 12288 inputs,
    all 4096 rows."""
    x, _ = c3_inputs(linear, m=4096)
    q, s = _gpu_quant(x)
    rq, rs = quant_rows_par(x)
    check_bytes(s.view(np.uint32), rs.view(np.uint32), "c3 x scales")
    check_bytes(q, rq, "c3 x codes")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("linear", [0, 6])
def test_c5_activations_all_rows(linear):
    """The stress chunk's K = 4096 and K = 12288 inputs, all 16384 rows: codes
    and scales bit-exact; zero rows give scale 0 and +0 codes; the
    saturating rows carry many +-448 codes."""
    m = 16384
    k = LAYER_SHAPES[linear][2]
    x = c5_x(m, k, linear)
    q, s = _gpu_quant(x)
    rq, rs = quant_rows_par(x)
    check_bytes(s.view(np.uint32), rs.view(np.uint32), "c5 x scales")
    check_bytes(q, rq, "c5 x codes")
    zero, big, heavy = c5_rows(m)
    assert np.all(s[zero] == 0) and np.all(q[zero] == 0)
    assert np.mean((q[heavy] & 0x7F) == 0x7E) > 0.05


@pytest.mark.parametrize("m,k,ld", [(1, 8, 8), (3, 24, 32), (5, 520, 528),
                                    (7, 4104, 4104), (2, 16392, 16400),
                                    (9, 12288, 12296), (33, 40000, 40000)])
def test_ragged_and_strided(m, k, ld):
    rng = np.random.default_rng(m * 7 + k)
    full = bf16_from_f64(rng.standard_normal((m, ld)) * 10.0 ** rng.uniform(-3, 3, (m, 1)))
    x = to_dev_bf16(full)[:, :k]
    q, s = fq.quantize_act_per_token(x)
    torch.cuda.synchronize()
    _check_rows(full[:, :k], host_bits(q), host_bits(s), what=f"ragged {m}x{k}")


def test_tiny_zero_and_negative_zero_rows():
    rows = np.zeros((4, 64), np.uint16)
    rows[0, :] = 0x8000                                  # all -0
    rows[1, 5] = 0x0001                                  # smallest subnormal
    rows[1, 6] = 0x8002
    rows[2, :] = bf16_from_f64(np.linspace(-2.0 ** -128, 2.0 ** -129, 64))
    rows[3, :8] = bf16_from_f64(np.array([1e-40, -1e-40, 5e-39, 0, 1, -1, 2, -448]) * 1e-30)
    q, s = _gpu_quant(rows)
    _check_rows(rows, q, s, what="tiny")
    assert np.all(q[0] == 0x80) and s[0] == 0


def test_deterministic():
    x, _ = c3_inputs(1, m=1024)
    a = _gpu_quant(x)
    b = _gpu_quant(x)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("split", ["1", "2", "4"])
@pytest.mark.parametrize("m,k,ld", [(1, 8, 8), (3, 520, 528), (7, 4104, 4104),
                                    (64, 4096, 4096), (5, 12288, 12296), (33, 1032, 1040),
                                    (130, 16392, 16400)])
def test_rows_split_over_waves(split, m, k, ld, monkeypatch):
    """Rows shared by 2 or 4 waves (the few-row variant): the waves' maxima
    meet in LDS, each wave quantizes its interleaved vectors; codes and
    scales bit-exact against the oracle for ragged and strided rows, a zero
    row and rows of very different magnitudes."""
    monkeypatch.setenv("FP8W8A8_QUANT_SPLIT", split)
    rng = np.random.default_rng(m * 13 + k)
    full = bf16_from_f64(rng.standard_normal((m, ld)) * 10.0 ** rng.uniform(-30, 30, (m, 1)))
    full[m // 2, :] = 0
    x = to_dev_bf16(full)[:, :k]
    q, s = fq.quantize_act_per_token(x)
    torch.cuda.synchronize()
    _check_rows(full[:, :k], host_bits(q), host_bits(s), what=f"split {split} {m}x{k}")


@pytest.mark.parametrize("seed", [0, 1])
def test_quantize_act_group_matches_oracle_and_single_calls(seed):
    """Several matrices in one launch (fp8w8a8_quantize_act_group): every
    item's codes and scales bit-exact against the oracle and against
    quantize_act_per_token on it alone; rows of K = 8 .. 16384 (ragged tails
    of a 16-byte step), 0 .. 300 rows, zero and large rows, a strided x."""
    rng = np.random.default_rng(900 + seed)
    shapes = [(1, 4096), (4, 12288), (3, 16384), (64, 4104), (0, 256), (300, 8),
              (17, 1024), (8, 2056)]
    xs_bits, xs = [], []
    for m, k in shapes:
        xf = rng.standard_normal((m, k)) * (10.0 ** rng.uniform(-3, 3, size=(m, 1)))
        if m >= 3:
            xf[1] = 0.0
            xf[2] *= 1e4
        bits = bf16_from_f64(xf)
        xs_bits.append(bits)
        xs.append(to_dev_bf16(bits) if m > 0 else
                  torch.empty((0, k), dtype=torch.bfloat16, device="cuda"))
    # One item read through a row stride larger than its row.
    wide = to_dev_bf16(bf16_from_f64(rng.standard_normal((5, 1024 + 64))))
    xs.append(wide[:, :1024])
    xs_bits.append(host_bits(wide)[:, :1024])
    outs = fq.quantize_act_group(xs)
    torch.cuda.synchronize()
    for i, (bits, x, (q, s)) in enumerate(zip(xs_bits, xs, outs)):
        rq, rs = oracle.quant_act_ref(bits)
        check_bytes(host_bits(s).view(np.uint32), rs.view(np.uint32), f"group quant {i} scales")
        check_bytes(host_bits(q), rq, f"group quant {i} codes")
        if x.shape[0] > 0:
            q1, s1 = fq.quantize_act_per_token(x)
            torch.cuda.synchronize()
            check_bytes(host_bits(q), host_bits(q1), f"group quant {i} vs single")
            check_bytes(host_bits(s).view(np.uint32), host_bits(s1).view(np.uint32),
                        f"group quant {i} scales vs single")
