"""Seeded generators for the five workloads of the FP8_DYNAMIC Linear.

The shapes are those of the quantized Linears of MOSS-VL's language model:
hidden size 4096 with 32 query heads and 8 key/value heads (MOSS-VL
architecture article, "overall architecture" section), hence head size 128
and k/v width 8 * 128 = 1024; the projections q, k, v, o, gate, up, down of
each self-attention layer are the ones the FP8-Dynamic recipe quantizes
(MOSS-VL quantization README, "FP8-Dynamic" recipe).  The MLP width is not on
the pages; 12288 is a synthetic choice.

Every draw comes from ``numpy.random.default_rng`` with an explicit seed.
Draws are float32, are scaled in float32, and are rounded to bfloat16 with
round-to-nearest-even on the bit pattern.  Arrays returned are ``uint16``
bfloat16 bit patterns, row-major.

Workloads (the benchmark and parity tests stand in for the pages' video
benchmarks, whose data and weights are not available, with synthetic data of
the model's Linear shapes and of the token counts those workloads produce):

* c1: one q_proj Linear, 16 tokens; X ~ N(0,1) with 1 % of entries x20;
  W ~ N(0, 0.02); seed 0 (X drawn first, then W).
* c2: one decode step through the 7 Linears at M in {1, 4, 8}; X as c1 with
  its own seed per Linear and M; W ~ N(0, 0.02).
* c3: a 4096-token prefill chunk through the 7 Linears;
  X[m, k] ~ N(0,1) * g[k], g[k] = 10^U(-1, 1) (outlier input channels).
* c4: 36 layers x 7 Linears with distinct weights at M in {64, 256};
  the first layer's input is drawn like c2, later inputs are the previous
  layer's outputs (see the tests).
* c5: a 16384-token prefill; X Student-t with 3 degrees of freedom, 0.1 % of
  rows all +0 (row 0 always), 0.1 % of rows x1e4, 0.1 % of rows with 10 % of
  their entries set to +-(row amax).
* swiglu: gate_up_proj's output ahead of the activation: gate ~ 1.5 N(0,1)
  with 1 % of entries x10, up ~ 1.5 N(0,1) (the spread of a K = 4096 dot
  product of c3-like activations with N(0, 0.02) weights).
* kv: K or V rows of the cache, kv_heads x head_dim = 1024 wide:
  N(0,1) x 10^U(-0.5, 0.5) per channel (k_proj / v_proj outputs with
  channels of different spread).
* norm: the RMSNorm input ahead of q/k/v and gate/up: residual-stream rows
  X[m, k] ~ N(0,1) * g[k], g[k] = 10^U(-1, 1) (outlier channels, as c3), and
  the norm weight gamma[k] ~ N(1, 0.25).
"""

import math

import numpy as np

HIDDEN = 4096
INTERMEDIATE = 12288
KV_WIDTH = 8 * (HIDDEN // 32)          # 8 KV heads x head size 128

#: (name, N = out features, K = in features) of the 7 quantized Linears.
LAYER_SHAPES = (
    ("q_proj", HIDDEN, HIDDEN),
    ("k_proj", KV_WIDTH, HIDDEN),
    ("v_proj", KV_WIDTH, HIDDEN),
    ("o_proj", HIDDEN, HIDDEN),
    ("gate_proj", INTERMEDIATE, HIDDEN),
    ("up_proj", INTERMEDIATE, HIDDEN),
    ("down_proj", HIDDEN, INTERMEDIATE),
)
LINEAR_NAMES = tuple(s[0] for s in LAYER_SHAPES)
N_SELF_ATTN_LAYERS = 36
ROLE_X, ROLE_W, ROLE_GAMMA = 0, 1, 2
CFG_NORM = 6
CFG_SWIGLU = 7
CFG_KV = 8


def rng_for(cfg: int, a: int, b: int, role: int) -> np.random.Generator:
    """Independent stream per (workload, index, index, role)."""
    return np.random.default_rng([cfg, a, b, role])


def bf16_from_f64(a: np.ndarray) -> np.ndarray:
    """Round to float32, then to bfloat16 bits (nearest, ties to even)."""
    f = np.ascontiguousarray(np.asarray(a).astype(np.float32))
    if not np.all(np.isfinite(f)):
        raise ValueError("generators only produce finite values")
    u = f.view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (r >> np.uint32(16)).astype(np.uint16)


def normal_bf16(rng, shape, std=1.0) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return bf16_from_f64(x)


def outlier_act_bf16(rng, shape, frac=0.01, factor=20.0) -> np.ndarray:
    """N(0,1) with an independent Bernoulli(frac) mask multiplied by factor."""
    x = rng.standard_normal(shape, dtype=np.float32)
    mask = rng.random(shape, dtype=np.float32) < np.float32(frac)
    x[mask] *= np.float32(factor)
    return bf16_from_f64(x)


def weight_bf16(cfg: int, layer: int, linear: int, n: int, k: int, rows=None):
    """W[n, k] ~ N(0, 0.02) for one Linear (or only its first `rows` rows,
    which are the same numbers: draws are made row by row)."""
    return normal_bf16(rng_for(cfg, layer, linear, ROLE_W),
                       (n if rows is None else rows, k), 0.02)


def c1_inputs():
    """(x [16, 4096], w [4096, 4096]) bf16 bits, seed 0, X drawn first."""
    rng = np.random.default_rng(0)
    x = outlier_act_bf16(rng, (16, HIDDEN))
    w = normal_bf16(rng, (HIDDEN, HIDDEN), 0.02)
    return x, w


def c2_inputs(m: int, linear: int):
    """(x [m, K], w [N, K]) for one Linear of the decode step."""
    _, n, k = LAYER_SHAPES[linear]
    x = outlier_act_bf16(rng_for(2, m, linear, ROLE_X), (m, k))
    w = weight_bf16(2, 0, linear, n, k)
    return x, w


def c3_x(m: int, k: int, seed_linear: int, rows=None) -> np.ndarray:
    """X[m, k] of the prefill chunk (or only its first `rows` rows)."""
    rng = rng_for(3, m, seed_linear, ROLE_X)
    gain = np.power(np.float32(10.0),
                    rng.uniform(-1.0, 1.0, size=k).astype(np.float32))
    x = rng.standard_normal((m if rows is None else rows, k),
                            dtype=np.float32) * gain[None, :]
    return bf16_from_f64(x)


def c3_inputs(linear: int, m: int = 4096):
    """(x [m, K], w [N, K]) for one Linear of the prefill chunk."""
    _, n, k = LAYER_SHAPES[linear]
    return c3_x(m, k, linear), weight_bf16(3, 0, linear, n, k)


def c4_x0(m: int) -> np.ndarray:
    """First-layer input of the 36-layer stack, drawn like c2."""
    return outlier_act_bf16(rng_for(4, m, 0, ROLE_X), (m, HIDDEN))


def c4_weight(layer: int, linear: int):
    _, n, k = LAYER_SHAPES[linear]
    return weight_bf16(4, layer, linear, n, k)


def c5_rows(m: int):
    """Row indices of the special rows of c5: (zero, big, amax-heavy)."""
    rng = rng_for(5, m, 99, ROLE_X)
    n_special = max(1, int(math.ceil(0.001 * m)))
    perm = rng.permutation(np.arange(1, m))
    zero = np.sort(np.concatenate([[0], perm[:n_special - 1]])).astype(np.int64)
    big = np.sort(perm[n_special:2 * n_special]).astype(np.int64)
    heavy = np.sort(perm[2 * n_special:3 * n_special]).astype(np.int64)
    return zero, big, heavy


def c5_x(m: int, k: int, seed_linear: int) -> np.ndarray:
    """Student-t(3) activations with the zero / large / saturating rows."""
    rng = rng_for(5, m, seed_linear, ROLE_X)
    z = rng.standard_normal((m, k), dtype=np.float32)
    # t_3 = Z / sqrt(V / 3) with V ~ chi-square(3) = 2 * Gamma(3/2).
    v = np.float32(2.0) * rng.standard_gamma(1.5, size=(m, k), dtype=np.float32)
    x = z / np.sqrt(v / np.float32(3.0))
    zero, big, heavy = c5_rows(m)
    x[zero] = 0.0
    x[big] *= np.float32(1e4)
    for r in heavy:
        amax = np.max(np.abs(x[r]))
        pick = rng.random(k) < 0.10
        sign = np.where(rng.random(k) < 0.5, -1.0, 1.0).astype(np.float32)
        x[r, pick] = sign[pick] * amax
    return bf16_from_f64(x)


def c5_inputs(linear: int, m: int = 16384):
    _, n, k = LAYER_SHAPES[linear]
    return c5_x(m, k, linear), weight_bf16(5, 0, linear, n, k)


def norm_inputs(m: int, k: int = HIDDEN, seed: int = 0):
    """(x [m, k], gamma [k]) bf16 bits for the RMSNorm ahead of a Linear."""
    rng = rng_for(CFG_NORM, seed, k, ROLE_X)
    ch = np.power(np.float32(10.0), rng.uniform(-1.0, 1.0, k).astype(np.float32))
    x = rng.standard_normal((m, k), dtype=np.float32) * ch[None, :]
    gamma = rng_for(CFG_NORM, seed, k, ROLE_GAMMA).standard_normal(k, dtype=np.float32)
    return bf16_from_f64(x), bf16_from_f64(np.float32(1.0) + np.float32(0.25) * gamma)


def swiglu_inputs(m: int, n: int, seed: int = 0):
    """(gate [m, n], up [m, n]) bf16 bits: the two halves of gate_up_proj's
    output for m tokens."""
    rng = rng_for(CFG_SWIGLU, seed, n, ROLE_X)
    g = rng.standard_normal((m, n), dtype=np.float32) * np.float32(1.5)
    g[rng.random((m, n), dtype=np.float32) < np.float32(0.01)] *= np.float32(10.0)
    u = rng_for(CFG_SWIGLU, seed, n, ROLE_W).standard_normal((m, n), dtype=np.float32)
    return bf16_from_f64(g), bf16_from_f64(u * np.float32(1.5))


def kv_inputs(t: int, width: int = KV_WIDTH, seed: int = 0):
    """K or V rows [t, width] bf16 bits for t tokens."""
    rng = rng_for(CFG_KV, seed, width, ROLE_X)
    ch = np.power(np.float32(10.0), rng.uniform(-0.5, 0.5, width).astype(np.float32))
    return bf16_from_f64(rng.standard_normal((t, width), dtype=np.float32) * ch[None, :])
