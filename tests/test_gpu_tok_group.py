"""The grouped call on given codes at a few tokens (fp8w8a8_fp8_linear_group,
1 <= M <= 256 tokens, up to 16 Linears in one launch; 16, 32, 48, 64, 128 or
256 token rows per unit, in stages of 512, 256 or 128 K bytes) and the
weight tiling it reads (fp8w8a8_tile_weights).

The tiling is bit-exact against oracle.tile_weights_ref.  Every item's
output is held to the elementwise tolerance of oracle.check against the
oracle's Linear on the same codes, computed on the row-major weights: the
activations are the oracle's own per-token quantization of seeded bf16 rows
(uploaded), the weights the GPU quantizer's codes (bit-exact against the
oracle in the weight tests), read back, and tiled on the GPU for the call.  The outputs are also bit-identical between two
runs and between persistent grids of different sizes: each output is one
thread's sum over K in ascending 128-value blocks whichever workgroup takes
its unit.

Cases: layer 0 of the 36-layer stack at M = 64 (q, k, v, o, gate, up on
one shared code buffer in one launch; down on the oracle's codes of the
GPU's up output), the decode layer's seven Linears at M = 4 and 8 in one
launch after one grouped quantization, ragged shapes at M = 1 .. 64 (N = 64, K with a partial
last 512-byte stage, tokens past the last full block of 16, zero and large
rows; 65-256 tokens in 128- and 256-row units), 16 items at the largest K,
and the tiling alone on its edge shapes.

fp8w8a8_fp8_linear_group_requant (one item's K summed in ranges, its output
re-quantized): that item's output within the oracle's tolerance and its
codes and scales bit-exact against the oracle's quantization of the GPU's
output, the other items bit-identical to the grouped call without it; on
layer 0 of the stack at M = 64 (down beside k and v, 1 to 8 ranges) and on
ragged items.
"""

import numpy as np
import pytest
import torch

import fp8_w8a8_dynamic_amd as fq
import oracle
from oracle import check_bytes, check_close
from tests.gpu_util import host_bits, to_dev_bf16, to_dev_f32, to_dev_u8
from workloads import LAYER_SHAPES, bf16_from_f64
from workloads.generators import c2_inputs, c4_weight, c4_x0, outlier_act_bf16

pytestmark = pytest.mark.gpu

UP = 5


def _codes(x_bits):
    """The oracle's per-token codes and scales of x, on the host and the GPU."""
    qx, sx = oracle.quant_act_ref(x_bits)
    return (qx, sx), (to_dev_u8(qx), to_dev_f32(sx))


def _weights(w_bits):
    """GPU-quantized weights (tiled for the call) and their host copies
    (row-major); the tiling checked bit-exact against the oracle's."""
    qw, sw = fq.quantize_weight_channelwise(to_dev_bf16(w_bits))
    tiled = fq.tile_weights(qw)
    hq = host_bits(qw)
    check_bytes(host_bits(tiled), oracle.tile_weights_ref(hq), "tiled weights")
    return (tiled, sw, qw.shape[0]), (hq, host_bits(sw))


def _group(acts, weights, outs=None):
    return fq.fp8_linear_group([a[1][0] for a in acts], [a[1][1] for a in acts],
                               [w[0][0] for w in weights], [w[0][1] for w in weights],
                               [w[0][2] for w in weights], outs=outs)


def _run_and_check(acts, weights, what):
    """acts[i] = ((qx, sx) host, (qx, sx) device); weights[i] likewise
    (device first).  Runs the group, checks every item against the oracle,
    returns the outputs' bits."""
    ys = _group(acts, weights)
    torch.cuda.synchronize()
    out = []
    for i, (a, w) in enumerate(zip(acts, weights)):
        y = host_bits(ys[i])
        check_close(y, oracle.linear_ref(a[0][0], a[0][1], w[1][0], w[1][1]),
                    f"{what} item {i}")
        out.append(y)
    return out


@pytest.mark.timeout(600)
def test_stack_layer0_m64():
    """Layer 0 of the 36-layer stack at M = 64: the six Linears that read
    the layer input in one launch on one shared code buffer, then down."""
    m = 64
    x = c4_x0(m)
    a = _codes(x)
    ws = [_weights(c4_weight(0, j)) for j in range(6)]
    ys = _run_and_check([a] * 6, ws, "stack layer 0, M = 64")
    up_bits = ys[UP]
    wd = _weights(c4_weight(0, 6))
    _run_and_check([_codes(up_bits)], [wd], "stack layer 0 down, M = 64")
    assert [y.shape for y in ys] == [(m, s[1]) for s in LAYER_SHAPES[:6]]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("m", [4, 8])
def test_decode_layer_grouped(m):
    """The decode layer at a few tokens in two launches: the seven Linears'
    inputs quantized by one quantize_act_group call, then the seven Linears
    on their codes in one grouped launch.  The 608 units of 64 rows exceed
    the 512-workgroup grid, so a second round is dealt (shifted past the 64
    workgroups that hold down's longer units).  Codes and scales bit-exact
    against the oracle's, outputs within its tolerance, and every output
    bit-identical to the same Linear alone in a one-item group (one round)."""
    xs, ws = [], []
    for j in range(7):
        x, w = c2_inputs(m, j)
        xs.append(x)
        ws.append(_weights(w))
    qs = fq.quantize_act_group([to_dev_bf16(x) for x in xs])
    refs = [oracle.quant_act_ref(x) for x in xs]
    for j, ((q, sc), (rq, rs)) in enumerate(zip(qs, refs)):
        check_bytes(host_bits(q), rq, f"decode M = {m} codes {j}")
        check_bytes(host_bits(sc).view(np.uint32), rs.view(np.uint32),
                    f"decode M = {m} scales {j}")
    ys = fq.fp8_linear_group([q for q, _ in qs], [sc for _, sc in qs],
                             [w[0][0] for w in ws], [w[0][1] for w in ws],
                             [w[0][2] for w in ws])
    torch.cuda.synchronize()
    for j, (y, w, r) in enumerate(zip(ys, ws, refs)):
        name = f"decode M = {m} {LAYER_SHAPES[j][0]}"
        yb = host_bits(y)
        check_close(yb, oracle.linear_ref(r[0], r[1], w[1][0], w[1][1]), name)
        alone = fq.fp8_linear_group([qs[j][0]], [qs[j][1]], [w[0][0]], [w[0][1]], [w[0][2]])
        torch.cuda.synchronize()
        check_bytes(host_bits(alone[0]), yb, f"{name}: grouped against alone")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("m", [4, 8])
def test_decode_layer_grouped_down_split(m):
    """The decode layer at a few tokens as the bench's grouped leg runs it:
    the seven Linears in one launch with down's K summed in ranges (units of
    their own beside the other six, then added in order by one more
    kernel, no re-quantization).  Every output within the oracle's
    tolerance; the six others bit-identical to the unsplit grouped call."""
    xs, ws = [], []
    for j in range(7):
        x, w = c2_inputs(m, j)
        xs.append(x)
        ws.append(_weights(w))
    refs = [oracle.quant_act_ref(x) for x in xs]
    acts = [(r, (to_dev_u8(r[0]), to_dev_f32(r[1]))) for r in refs]
    ys, qy, sy = fq.fp8_linear_group_requant(
        [a[1][0] for a in acts], [a[1][1] for a in acts], [w[0][0] for w in ws],
        [w[0][1] for w in ws], [w[0][2] for w in ws], 6, requant=False)
    torch.cuda.synchronize()
    assert qy is None and sy is None
    base = _group(acts, ws)
    torch.cuda.synchronize()
    for j, (y, w, r) in enumerate(zip(ys, ws, refs)):
        name = f"decode M = {m} {LAYER_SHAPES[j][0]}, down split"
        yb = host_bits(y)
        check_close(yb, oracle.linear_ref(r[0], r[1], w[1][0], w[1][1]), name)
        if j != 6:
            check_bytes(yb, host_bits(base[j]), f"{name}: against the unsplit call")


WIDE = [(128, 640), (256, 640), (1024, 1152), (128, 4224), (384, 12288),
        (4096, 512), (128, 128)]
NARROW = [(64, 640), (192, 640), (320, 4224), (64, 128), (1024, 12288)]


def _ragged_inputs(m, seed, shapes):
    """Items of assorted shapes; items 0 and 1 share one code buffer."""
    rng = np.random.default_rng(700 + seed)
    acts, weights = [], []
    shared = None
    for i, (n, k) in enumerate(shapes):
        if i == 1:
            acts.append(shared)
        else:
            xf = rng.standard_normal((m, k)) * (10.0 ** rng.uniform(-3, 3, size=(m, 1)))
            xf *= np.where(rng.random((m, k)) < 0.01, 20.0, 1.0)
            if m >= 5:
                xf[1] = 0.0          # a zero row: scale 0, codes 0, output 0
                xf[3] *= 1e4         # a large row
            a = _codes(bf16_from_f64(xf))
            acts.append(a)
            if i == 0:
                shared = a
        weights.append(_weights(bf16_from_f64(rng.standard_normal((n, k)) * 0.02)))
    return acts, weights


@pytest.mark.parametrize("m,shapes", [(m, "wide") for m in (1, 5, 16, 17, 33, 63, 64)]
                         + [(m, "narrow") for m in (3, 40, 64)]
                         + [(m, "wide") for m in (65, 128, 129, 200, 256)]
                         + [(m, "narrow") for m in (100, 256)])
def test_ragged_shapes(m, shapes, monkeypatch):
    acts, weights = _ragged_inputs(m, m, WIDE if shapes == "wide" else NARROW)
    base = _run_and_check(acts, weights, f"ragged {shapes} M = {m}")
    # The same bits on a persistent grid of 1, 2 and 7 workgroups (hundreds
    # of units each, the pipeline running across unit boundaries), with
    # the weights requested three stages ahead instead of two, with the
    # codes one and two stages ahead, and (33-64 tokens) without the
    # rolling refill of the weights.
    for key, val in (("FP8W8A8_TOKG_GRID", "1"), ("FP8W8A8_TOKG_GRID", "2"),
                     ("FP8W8A8_TOKG_GRID", "7"), ("FP8W8A8_TOKG_DEPTH", "3"),
                     ("FP8W8A8_TOKG_CODES", "1"), ("FP8W8A8_TOKG_CODES", "2"),
                     ("FP8W8A8_TOKG_ROLL", "0")):
        monkeypatch.setenv(key, val)
        ys = _group(acts, weights)
        torch.cuda.synchronize()
        monkeypatch.delenv(key)
        for i, y in enumerate(ys):
            check_bytes(host_bits(y), base[i],
                        f"ragged {shapes} M = {m} {key}={val} item {i}")


def test_sixteen_items_largest_k():
    """16 items of N = 64 (one 64-row unit each) at K = 16384, M = 64, each
    with its own codes; run twice, same bits."""
    m = 64
    rng = np.random.default_rng(77)
    acts = [_codes(outlier_act_bf16(rng, (m, 16384))) for _ in range(16)]
    weights = [_weights(bf16_from_f64(rng.standard_normal((64, 16384)) * 0.02))
               for _ in range(16)]
    first = _run_and_check(acts, weights, "16 items K = 16384")
    again = _run_and_check(acts, weights, "16 items K = 16384, again")
    for i in range(16):
        check_bytes(again[i], first[i], f"16 items run twice item {i}")


def test_outputs_into_given_buffers():
    """outs= given: results land in the caller's tensors, others untouched."""
    m, rng = 24, np.random.default_rng(9)
    a = _codes(outlier_act_bf16(rng, (m, 1024)))
    w = _weights(bf16_from_f64(rng.standard_normal((256, 1024)) * 0.02))
    big = torch.full((m + 2, 256), 7.0, dtype=torch.bfloat16, device="cuda")
    out = big[1:m + 1]
    _group([a], [w], outs=[out])
    torch.cuda.synchronize()
    check_close(host_bits(out), oracle.linear_ref(a[0][0], a[0][1], w[1][0], w[1][1]),
                "outs given")
    assert torch.all(big[0] == 7.0) and torch.all(big[m + 1] == 7.0)


@pytest.mark.parametrize("n,k", [(16, 128), (48, 384), (32, 640), (64, 1408), (4096, 4096),
                                 (1024, 12288), (80, 16384)])
def test_tile_weights_bit_exact(n, k):
    qw = torch.from_numpy(np.random.default_rng(n + k).integers(
        0, 256, size=(n, k), dtype=np.uint8)).to("cuda")
    t = fq.tile_weights(qw)
    torch.cuda.synchronize()
    check_bytes(host_bits(t), oracle.tile_weights_ref(host_bits(qw)), f"tile {n}x{k}")


def _requant_check(ys, qy, sy, acts, weights, rq, what):
    """Item rq's y within the oracle's tolerance and its codes and scales
    bit-exact against the oracle's quantization of that y; returns every
    item's output bits."""
    out = []
    for i, (y, a, w) in enumerate(zip(ys, acts, weights)):
        yb = host_bits(y)
        check_close(yb, oracle.linear_ref(a[0][0], a[0][1], w[1][0], w[1][1]),
                    f"{what} item {i}")
        out.append(yb)
    rq_codes, rq_scales = oracle.quant_act_ref(out[rq])
    check_bytes(host_bits(qy), rq_codes, f"{what} codes of item {rq}")
    check_bytes(host_bits(sy).view(np.uint32), rq_scales.view(np.uint32),
                f"{what} scales of item {rq}")
    return out


@pytest.mark.timeout(600)
def test_group_requant_stack_layer0_m64(monkeypatch):
    """Layer 0 of the stack at M = 64 as the bench's grouped leg runs its
    second launch: down (K = 12288, its K summed in ranges that are units
    of their own) beside k and v, down's output re-quantized.  down within
    tolerance of the oracle, its codes and scales bit-exact against the
    oracle's quantization of the GPU's down output; k and v bit-identical
    to the grouped call without down (each output one thread's sum over K).
    The same for every range count from 1 to 8 (test hook), and bit-equal
    on a second run."""
    m = 64
    x = c4_x0(m)
    a = _codes(x)
    wk, wv = _weights(c4_weight(0, 1)), _weights(c4_weight(0, 2))
    ref_kv = _group([a, a], [wk, wv])
    torch.cuda.synchronize()
    ref_kv = [host_bits(t) for t in ref_kv]
    wu = _weights(c4_weight(0, UP))
    up = _group([a], [wu])[0]
    torch.cuda.synchronize()
    au = _codes(host_bits(up))
    wd = _weights(c4_weight(0, 6))
    acts, weights = [au, a, a], [wd, wk, wv]

    def run():
        ys, qy, sy = fq.fp8_linear_group_requant(
            [t[1][0] for t in acts], [t[1][1] for t in acts], [w[0][0] for w in weights],
            [w[0][1] for w in weights], [w[0][2] for w in weights], 0)
        torch.cuda.synchronize()
        return ys, qy, sy

    base = _requant_check(*run(), acts, weights, 0, "group requant M = 64")
    for i in (1, 2):
        check_bytes(base[i], ref_kv[i - 1], f"group requant M = 64 item {i} against alone")
    again = _requant_check(*run(), acts, weights, 0, "group requant M = 64, again")
    check_bytes(again[0], base[0], "group requant M = 64 run twice")
    for s in (1, 2, 3, 4, 6, 8):
        monkeypatch.setenv("FP8W8A8_TOKG_SPLITS", str(s))
        got = _requant_check(*run(), acts, weights, 0, f"group requant M = 64, {s} ranges")
        monkeypatch.delenv("FP8W8A8_TOKG_SPLITS")
        for i in (1, 2):
            check_bytes(got[i], ref_kv[i - 1], f"{s} ranges item {i} against alone")


@pytest.mark.parametrize("m", [1, 5, 17, 33, 64, 96, 256])
@pytest.mark.parametrize("rq", [0, 2])
def test_group_requant_ragged(m, rq, monkeypatch):
    """Ragged items (zero and large token rows, K with a partial last
    512-byte stage, N = 64) with the re-quantized item first or last; the
    same bits on a persistent grid of 1 and 7 workgroups, with the codes
    one and two stages ahead and without the rolling refill."""
    # (Items 0 and 1 share one code buffer, so they share K.)
    shapes = ([(320, 1536), (64, 1536), (1024, 1152)] if rq == 0
              else [(64, 640), (192, 640), (384, 1536)])
    acts, weights = _ragged_inputs(m, 40 + m + rq, shapes)
    def run():
        ys, qy, sy = fq.fp8_linear_group_requant(
            [t[1][0] for t in acts], [t[1][1] for t in acts], [w[0][0] for w in weights],
            [w[0][1] for w in weights], [w[0][2] for w in weights], rq)
        torch.cuda.synchronize()
        return ys, qy, sy
    base = _requant_check(*run(), acts, weights, rq, f"ragged requant M = {m}")
    alone = _group([a for i, a in enumerate(acts) if i != rq],
                   [w for i, w in enumerate(weights) if i != rq])
    torch.cuda.synchronize()
    others = [i for i in range(3) if i != rq]
    for i, y in zip(others, alone):
        check_bytes(base[i], host_bits(y), f"ragged requant M = {m} item {i} against alone")
    for key, val in (("FP8W8A8_TOKG_GRID", "1"), ("FP8W8A8_TOKG_GRID", "7"),
                     ("FP8W8A8_TOKG_CODES", "1"), ("FP8W8A8_TOKG_CODES", "2"),
                     ("FP8W8A8_TOKG_ROLL", "0")):
        monkeypatch.setenv(key, val)
        got = _requant_check(*run(), acts, weights, rq, f"ragged requant M = {m} {key}={val}")
        monkeypatch.delenv(key)
        for i in range(3):
            check_bytes(got[i], base[i], f"ragged requant M = {m} {key}={val} item {i}")
    # K ranges that start inside a 512-byte K panel of the tiled weights
    # (the split item has K = 1536, twelve K blocks: 2 ranges start at
    # blocks 0 and 6, 6 ranges at blocks 0, 2, ..., 10): the split item
    # within the tolerance, the others the same bits.
    for s in ("2", "6"):
        monkeypatch.setenv("FP8W8A8_TOKG_SPLITS", s)
        got = _requant_check(*run(), acts, weights, rq, f"ragged requant M = {m}, {s} ranges")
        monkeypatch.delenv("FP8W8A8_TOKG_SPLITS")
        for i in others:
            check_bytes(got[i], base[i], f"ragged requant M = {m}, {s} ranges, item {i}")
    # Without re-quantization: the same y (the ranges added in the same
    # order by the plain reduction), no codes.
    ys, qy, sy = fq.fp8_linear_group_requant(
        [t[1][0] for t in acts], [t[1][1] for t in acts], [w[0][0] for w in weights],
        [w[0][1] for w in weights], [w[0][2] for w in weights], rq, requant=False)
    torch.cuda.synchronize()
    assert qy is None and sy is None
    for i in range(3):
        check_bytes(host_bits(ys[i]), base[i], f"ragged split-only M = {m} item {i}")
