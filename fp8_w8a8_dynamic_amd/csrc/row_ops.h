// Per-row arithmetic of the fused pre-quantization steps, the BF16 RMSNorm
// ahead of q/k/v and gate/up and the SiLU-gated activation ahead of down
// (MOSS-VL-Realtime-FP8 article, component / precision map: both stay
// BF16 and feed FP8_DYNAMIC Linears).  Shared by their stand-alone kernels
// and by the decode GEMV's activation staging, so that a fused decode call
// and the two-step path give the same codes bit for bit.
#pragma once

#include "device_common.h"

namespace fp8w8a8 {

// ---- wave reductions -------------------------------------------------------

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL,
                                                    ROW_MASK, 0xf, false));
}

// Sum over the 64 lanes (the DPP pattern of wave_max_u32: lanes that a move
// does not write add the 0 it leaves).  Fixed order, so deterministic; the
// result is returned to every lane.
__device__ __forceinline__ float wave_sum_f32(float v) {
  v += dpp_f32<0xb1, 0xf>(v);
  v += dpp_f32<0x4e, 0xf>(v);
  v += dpp_f32<0x141, 0xf>(v);
  v += dpp_f32<0x140, 0xf>(v);
  v += dpp_f32<0x142, 0xa>(v);
  v += dpp_f32<0x143, 0xc>(v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// ---- RMSNorm -----------------------------------------------------------------
//
// The row's sum of squares has one fixed evaluation order, whatever the
// kernel layout: the row is cut into blocks of 512 values (64 lanes x 8,
// lane l holding values 8l .. 8l+7 of the block); a lane's partial is the
// v_dot2c_f32_bf16 chain over its 8 values from 0, a block's sum is the DPP
// tree over its 64 lanes, and the blocks are added in order from 0.

__device__ __forceinline__ uint32_t amax8_bits(uint4 v, uint32_t m) {
  m = pk_max_u16(m, bf16x2_abs_bits(v.x));
  m = pk_max_u16(m, bf16x2_abs_bits(v.y));
  m = pk_max_u16(m, bf16x2_abs_bits(v.z));
  m = pk_max_u16(m, bf16x2_abs_bits(v.w));
  return m;
}

// Row-uniform factor p = 2^-e from the row's amax bit pattern (15 bits).
__device__ __forceinline__ float pow2_for_amax(uint32_t amax_bits) {
  int e = static_cast<int>(amax_bits >> 7) - 127;
  e = e < -126 ? -126 : (e > 126 ? 126 : e);
  return __uint_as_float(static_cast<uint32_t>(127 - e) << 23);
}

typedef __bf16 bf16x2_dot_t __attribute__((ext_vector_type(2)));

// A lane's partial: two exact bf16 products per v_dot2c_f32_bf16.  Subnormal
// bf16 inputs may count as zero here; their squares are below 2^-252,
// negligible next to any sum this path keeps (at least 2^-60; smaller sums
// take the exactly scaled path below).
__device__ __forceinline__ float sumsq_lane(uint4 v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16x2_dot_t a = __builtin_bit_cast(bf16x2_dot_t, w[i]);
    s = __builtin_amdgcn_fdot2_f32_bf16(a, a, s, false);
  }
  return s;
}

// The same over x * p (p a power of two: each x * p is exact).
__device__ __forceinline__ float sumsq_lane_scaled(uint4 v, float p) {
  const float e[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                      bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s = __builtin_fmaf(e[i] * p, e[i] * p, s);
  return s;
}

// One block's sum (every lane of the wave holds one vector of the block).
__device__ __forceinline__ float block_sumsq(uint4 v) {
  return wave_sum_f32(sumsq_lane(v));
}
__device__ __forceinline__ float block_sumsq_scaled(uint4 v, float p) {
  return wave_sum_f32(sumsq_lane_scaled(v, p));
}

// True when the row's float32 sum of squares is trustworthy unscaled.
__device__ __forceinline__ bool sumsq_in_range(float ss) {
  return ss >= 0x1p-60f && ss <= 0x1p127f;
}

// f with f * p = 1 / sqrt(mean(x^2) + eps), from the (scaled) sum of squares
// (float64 only for range: eps p^2 may exceed float32).
__device__ __forceinline__ float norm_factor(float ss, int64_t k, float eps,
                                             float p) {
  const float ms = ss / static_cast<float>(k);
  const double pd = static_cast<double>(p);
  const double d = __builtin_sqrt(static_cast<double>(ms) +
                                  static_cast<double>(eps) * pd * pd);
  return d > 0.0 ? static_cast<float>(1.0 / d) : 1.0f;
}

// Row-uniform factors, and whether p * f is a normal float (then x * (p f)
// is the same product as (x p) f).
struct NormFactor {
  float p, f, pf;
  bool one_mul;
};

__device__ __forceinline__ NormFactor make_norm_factor(float ss, int64_t k,
                                                       float eps, float p) {
  NormFactor n;
  n.p = p;
  n.f = norm_factor(ss, k, eps, p);
  n.pf = p * n.f;
  n.one_mul = n.pf >= 0x1p-126f && n.pf <= 0x1p127f;
  return n;
}

// t = bf16(x * c) (ONE_MUL) or bf16((x * p) * f), then y = bf16(gamma t)
// for two packed elements (the float32 product of two bf16 is exact, so y
// is rounded once); am accumulates max |gamma t|.
template <bool ONE_MUL>
__device__ __forceinline__ uint32_t norm2(uint32_t x, uint32_t g, float p,
                                          float f, float& am) {
  float a = bf16_lo(x), b = bf16_hi(x);
  if (ONE_MUL) {
    a *= f;
    b *= f;
  } else {
    a = (a * p) * f;
    b = (b * p) * f;
  }
  const uint32_t t = pack_bf16x2(a, b);
  const float ya = bf16_lo(g) * bf16_lo(t), yb = bf16_hi(g) * bf16_hi(t);
  am = __builtin_fmaxf(am, __builtin_fmaxf(__builtin_fabsf(ya), __builtin_fabsf(yb)));
  return pack_bf16x2(ya, yb);
}

template <bool ONE_MUL>
__device__ __forceinline__ uint4 norm8(uint4 x, uint4 g, float p, float f,
                                       float& am) {
  uint4 r;
  r.x = norm2<ONE_MUL>(x.x, g.x, p, f, am);
  r.y = norm2<ONE_MUL>(x.y, g.y, p, f, am);
  r.z = norm2<ONE_MUL>(x.z, g.z, p, f, am);
  r.w = norm2<ONE_MUL>(x.w, g.w, p, f, am);
  return r;
}

__device__ __forceinline__ uint4 norm8(uint4 x, uint4 g, const NormFactor& nf,
                                       float& am) {
  return nf.one_mul ? norm8<true>(x, g, 1.0f, nf.pf, am)
                    : norm8<false>(x, g, nf.p, nf.f, am);
}

// The row's scale from max |gamma t| over the row: the bf16 rounding is
// monotonic, so max |y| = bf16(max |gamma t|).
__device__ __forceinline__ float scale_from_row_max(float am) {
  return row_scale(__uint_as_float(static_cast<uint32_t>(f32_to_bf16_bits(am)) << 16));
}

// ---- SiLU-gated activation -------------------------------------------------
//
// s = bf16(silu(g)), h = bf16(s * u).  silu in float32: g * rcp(1 + 2^y),
// y = -g log2(e) (v_exp_f32, v_rcp_f32) for g >= -44; below, 1 + 2^y is 2^y
// to float32 precision and silu(g) = g e^g to 2^-63, evaluated as
// g * 2^-64 * 2^(g log2(e) + 64) so that no step underflows before the last
// (v_ldexp_f32 rounds into the subnormals correctly).  silu_any equals
// silu_common wherever g >= -44, so which form a caller applies to a slice
// changes no result.

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kSiluSplit = -44.0f;

__device__ __forceinline__ float silu_common(float g) {
  const float e = __builtin_amdgcn_exp2f(g * -kLog2e);
  return g * __builtin_amdgcn_rcpf(1.0f + e);
}

__device__ __forceinline__ float silu_any(float g) {
  const float t = g * kLog2e;
  const float deep = g * __builtin_ldexpf(__builtin_amdgcn_exp2f(t + 64.0f), -64);
  return g >= kSiluSplit ? silu_common(g) : deep;
}

template <bool COMMON>
__device__ __forceinline__ uint32_t swiglu2(uint32_t g2, uint32_t u2, float& am) {
  const float ga = bf16_lo(g2), gb = bf16_hi(g2);
  const uint32_t s = COMMON ? pack_bf16x2(silu_common(ga), silu_common(gb))
                            : pack_bf16x2(silu_any(ga), silu_any(gb));
  const float ha = bf16_lo(s) * bf16_lo(u2), hb = bf16_hi(s) * bf16_hi(u2);
  am = __builtin_fmaxf(am, __builtin_fmaxf(__builtin_fabsf(ha), __builtin_fabsf(hb)));
  return pack_bf16x2(ha, hb);
}

template <bool COMMON>
__device__ __forceinline__ uint4 swiglu8(uint4 g, uint4 u, float& am) {
  uint4 h;
  h.x = swiglu2<COMMON>(g.x, u.x, am);
  h.y = swiglu2<COMMON>(g.y, u.y, am);
  h.z = swiglu2<COMMON>(g.z, u.z, am);
  h.w = swiglu2<COMMON>(g.w, u.w, am);
  return h;
}

// Whether any of the 8 packed gate values is below kSiluSplit.
__device__ __forceinline__ bool any_deep8(uint4 g) {
  const float m = __builtin_fminf(
      __builtin_fminf(__builtin_fminf(bf16_lo(g.x), bf16_hi(g.x)),
                      __builtin_fminf(bf16_lo(g.y), bf16_hi(g.y))),
      __builtin_fminf(__builtin_fminf(bf16_lo(g.z), bf16_hi(g.z)),
                      __builtin_fminf(bf16_lo(g.w), bf16_hi(g.w))));
  return m < kSiluSplit;
}

}  // namespace fp8w8a8
