// BF16 RMSNorm fused with the per-token FP8 quantization of its output.
//
// In the quantized model the language model's norms are RMSNorm kept in
// BF16, and the Linears right after them (q/k/v after the input norm,
// gate/up after the post-attention norm) are FP8_DYNAMIC Linears whose first
// step quantizes each token's input row with its own scale
// (MOSS-VL-Realtime-FP8 article, component / precision map; MOSS-VL
// quantization README, "FP8-Dynamic").  The norm's output row is exactly the
// row whose amax that scale needs, so one kernel can normalize a row and
// quantize it while it is still in registers: x is read from HBM once, the
// codes and the scale are written once, and the bf16 norm output is written
// only when the caller asks for it.
//
// One wavefront owns one row of k elements (buffer loads and stores, whose
// descriptors clip the ragged tail; padding lanes hold zeros throughout):
//   1. ss = sum x^2 in float32 (per-lane sums, then a DPP tree); a row whose
//      sum leaves [2^-60, 2^127] (squares that underflow or overflow float32)
//      takes a rare path: p = 2^-e, e the (clamped) exponent of the row's
//      amax, every x p is exact and below 2 in magnitude, and ss is taken
//      over x p instead (p = 1 otherwise);
//   2. D = sqrt(ss / k + eps p^2) in float64 (range only: eps p^2 may exceed
//      float32), f = fl32(1 / D), so that f p = 1 / sqrt(mean(x^2) + eps);
//      an all-zero row with eps = 0 takes f = 1 (its output is x itself,
//      signed zeros);
//   3. t = bf16(x (p f)) when p f is a normal float (then x (p f) is the
//      same product as (x p) f), else bf16((x p) f); y = bf16(gamma t): two
//      bfloat16 roundings, as a BF16 norm produces them; the float32 product
//      of two bfloat16 values is exact, so y is rounded once from the exact
//      product, and max |y| is the rounding of the largest |gamma t|;
//   4. the per-token quantization of y, bit for bit as the stand-alone
//      quantizer (scale = amax / 448, correctly rounded quotients,
//      round-to-nearest-even, saturation at +-448).
// HBM traffic per row: 2k bytes in, k bytes of codes + 4 bytes of scale out
// (+ 2k bytes if y is stored); gamma (2k bytes, shared by all rows) is read
// from L2.
#include "device_common.h"
#include "launch.h"

namespace fp8w8a8 {

namespace detail {

constexpr int kNormRowsPerBlock = 4;  // 4 waves, one row each

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL,
                                                    ROW_MASK, 0xf, false));
}

// Sum over the 64 lanes (same DPP pattern as wave_max_u32: lanes that a
// move does not write add the 0 it leaves).  The order of the additions is
// fixed, so the result is deterministic.
__device__ __forceinline__ float wave_sum_f32(float v) {
  v += dpp_f32<0xb1, 0xf>(v);
  v += dpp_f32<0x4e, 0xf>(v);
  v += dpp_f32<0x141, 0xf>(v);
  v += dpp_f32<0x140, 0xf>(v);
  v += dpp_f32<0x142, 0xa>(v);
  v += dpp_f32<0x143, 0xc>(v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

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

__device__ __forceinline__ float sumsq8(uint4 v, float s) {
  s = __builtin_fmaf(bf16_lo(v.x), bf16_lo(v.x), s);
  s = __builtin_fmaf(bf16_hi(v.x), bf16_hi(v.x), s);
  s = __builtin_fmaf(bf16_lo(v.y), bf16_lo(v.y), s);
  s = __builtin_fmaf(bf16_hi(v.y), bf16_hi(v.y), s);
  s = __builtin_fmaf(bf16_lo(v.z), bf16_lo(v.z), s);
  s = __builtin_fmaf(bf16_hi(v.z), bf16_hi(v.z), s);
  s = __builtin_fmaf(bf16_lo(v.w), bf16_lo(v.w), s);
  return __builtin_fmaf(bf16_hi(v.w), bf16_hi(v.w), s);
}

__device__ __forceinline__ float sumsq8_scaled(uint4 v, float p, float s) {
  const float e[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                      bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
#pragma unroll
  for (int i = 0; i < 8; ++i) s = __builtin_fmaf(e[i] * p, e[i] * p, s);
  return s;
}

// True when the row's float32 sum of squares is trustworthy unscaled.
__device__ __forceinline__ bool sumsq_in_range(float ss) {
  return ss >= 0x1p-60f && ss <= 0x1p127f;
}

// f with f * p = 1 / sqrt(mean(x^2) + eps), from the (scaled) sum of squares.
__device__ __forceinline__ float norm_factor(float ss, int64_t k, float eps,
                                             float p) {
  const float ms = ss / static_cast<float>(k);
  const double pd = static_cast<double>(p);
  const double d = __builtin_sqrt(static_cast<double>(ms) +
                                  static_cast<double>(eps) * pd * pd);
  return d > 0.0 ? static_cast<float>(1.0 / d) : 1.0f;
}

// t = bf16(x * c) (ONE_MUL) or bf16((x * p) * f), then y = bf16(gamma t) for
// two packed elements; am accumulates max |gamma t|.
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

// The row's scale from max |gamma t| over the row: the bf16 rounding is
// monotonic, so max |y| = bf16(max |gamma t|).
__device__ __forceinline__ float scale_from_products(float am) {
  const uint32_t m = wave_max_u32(__float_as_uint(am));  // non-negative floats
  return row_scale(__uint_as_float(
      static_cast<uint32_t>(f32_to_bf16_bits(__uint_as_float(m))) << 16));
}

// Row-uniform factor p and whether p * f is a normal float.
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

template <int NV>
__global__ __launch_bounds__(256) void rmsnorm_quant_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int k, int64_t ldx,
    const uint16_t* __restrict__ gamma, float eps, uint8_t* __restrict__ q,
    float* __restrict__ scale, uint16_t* __restrict__ y, int64_t ldy) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kNormRowsPerBlock +
                      __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (row >= rows) return;
  const uint32_t row_bytes = static_cast<uint32_t>(k) * 2u;
  const auto src = row_rsrc(x + row * ldx, row_bytes);
  const auto gsrc = row_rsrc(gamma, row_bytes);
  uint4 v[NV], g[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) v[i] = buf_load16(src, (i * 64 + lane) * 16u);
#pragma unroll
  for (int i = 0; i < NV; ++i) g[i] = buf_load16(gsrc, (i * 64 + lane) * 16u);
  float ss = 0.0f;
#pragma unroll
  for (int i = 0; i < NV; ++i) ss = sumsq8(v[i], ss);
  ss = wave_sum_f32(ss);
  float p = 1.0f;
  if (!sumsq_in_range(ss)) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < NV; ++i) m = amax8_bits(v[i], m);
    p = pow2_for_amax(wave_max_u32(max(m & 0xffffu, m >> 16)));
    ss = 0.0f;
#pragma unroll
    for (int i = 0; i < NV; ++i) ss = sumsq8_scaled(v[i], p, ss);
    ss = wave_sum_f32(ss);
  }
  const NormFactor nf = make_norm_factor(ss, k, eps, p);
  float am = 0.0f;
  if (nf.one_mul) {
#pragma unroll
    for (int i = 0; i < NV; ++i) v[i] = norm8<true>(v[i], g[i], 1.0f, nf.pf, am);
  } else {
#pragma unroll
    for (int i = 0; i < NV; ++i) v[i] = norm8<false>(v[i], g[i], nf.p, nf.f, am);
  }
  const float s = scale_from_products(am);
  uint2 codes[NV];
  quantize_row<NV>(v, make_divisor(s), codes);
  const auto dst = row_rsrc(q + row * static_cast<int64_t>(k), static_cast<uint32_t>(k));
#pragma unroll
  for (int i = 0; i < NV; ++i) buf_store8(codes[i], dst, (i * 64 + lane) * 8u);
  if (y != nullptr) {
    const auto ydst = row_rsrc(y + row * ldy, row_bytes);
#pragma unroll
    for (int i = 0; i < NV; ++i) buf_store16(v[i], ydst, (i * 64 + lane) * 16u);
  }
  if (lane == 0) scale[row] = s;
}

// Rows longer than the register-resident variants: the same arithmetic in
// three passes over the row (sum of squares, amax of y, output; a fourth for
// the amax of x on the rare rescaled path), the later ones reading the row
// again from L2.  (x * 1) * (p f) is the same product as x * (p f).
__global__ __launch_bounds__(256) void rmsnorm_quant_long_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t k, int64_t ldx,
    const uint16_t* __restrict__ gamma, float eps, uint8_t* __restrict__ q,
    float* __restrict__ scale, uint16_t* __restrict__ y, int64_t ldy) {
  const int lane = threadIdx.x & 63;
  const int64_t row =
      static_cast<int64_t>(blockIdx.x) * kNormRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;
  const uint4* src = reinterpret_cast<const uint4*>(x + row * ldx);
  const uint4* gsrc = reinterpret_cast<const uint4*>(gamma);
  const int64_t nvec = k >> 3;
  float ss = 0.0f;
  for (int64_t idx = lane; idx < nvec; idx += 64) ss = sumsq8(src[idx], ss);
  ss = wave_sum_f32(ss);
  float p = 1.0f;
  if (!sumsq_in_range(ss)) {
    uint32_t m = 0;
    for (int64_t idx = lane; idx < nvec; idx += 64) m = amax8_bits(src[idx], m);
    p = pow2_for_amax(wave_max_u32(max(m & 0xffffu, m >> 16)));
    ss = 0.0f;
    for (int64_t idx = lane; idx < nvec; idx += 64)
      ss = sumsq8_scaled(src[idx], p, ss);
    ss = wave_sum_f32(ss);
  }
  const NormFactor nf = make_norm_factor(ss, k, eps, p);
  const float pa = nf.one_mul ? 1.0f : nf.p, fa = nf.one_mul ? nf.pf : nf.f;
  float am = 0.0f;
  for (int64_t idx = lane; idx < nvec; idx += 64)
    norm8<false>(src[idx], gsrc[idx], pa, fa, am);
  const float s = scale_from_products(am);
  const RowDivisor d = make_divisor(s);
  uint2* dst = reinterpret_cast<uint2*>(q + row * k);
  uint4* ydst = y != nullptr ? reinterpret_cast<uint4*>(y + row * ldy) : nullptr;
  for (int64_t idx = lane; idx < nvec; idx += 64) {
    const uint4 t = norm8<false>(src[idx], gsrc[idx], pa, fa, am);
    dst[idx] = quantize8(t, d);
    if (ydst != nullptr) ydst[idx] = t;
  }
  if (lane == 0) scale[row] = s;
}

template <int NV>
hipError_t launch_norm_nv(const uint16_t* x, int64_t rows, int64_t k,
                          int64_t ldx, const uint16_t* gamma, float eps,
                          uint8_t* q, float* scale, uint16_t* y, int64_t ldy,
                          hipStream_t stream) {
  const int64_t blocks = (rows + kNormRowsPerBlock - 1) / kNormRowsPerBlock;
  rmsnorm_quant_kernel<NV><<<dim3(static_cast<uint32_t>(blocks)), dim3(256), 0,
                             stream>>>(x, rows, static_cast<int>(k), ldx, gamma,
                                       eps, q, scale, y, ldy);
  return hipGetLastError();
}

}  // namespace detail
using namespace detail;

hipError_t launch_rmsnorm_quant(const uint16_t* x, int64_t rows, int64_t k,
                                int64_t ldx, const uint16_t* gamma, float eps,
                                uint8_t* q, float* scale, uint16_t* y,
                                int64_t ldy, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const int64_t per_lane = (k / 8 + 63) / 64;
  if (per_lane <= 1)
    return launch_norm_nv<1>(x, rows, k, ldx, gamma, eps, q, scale, y, ldy, stream);
  if (per_lane <= 2)
    return launch_norm_nv<2>(x, rows, k, ldx, gamma, eps, q, scale, y, ldy, stream);
  if (per_lane <= 4)
    return launch_norm_nv<4>(x, rows, k, ldx, gamma, eps, q, scale, y, ldy, stream);
  if (per_lane <= 8)
    return launch_norm_nv<8>(x, rows, k, ldx, gamma, eps, q, scale, y, ldy, stream);
  if (per_lane <= 12)
    return launch_norm_nv<12>(x, rows, k, ldx, gamma, eps, q, scale, y, ldy, stream);
  const int64_t blocks = (rows + kNormRowsPerBlock - 1) / kNormRowsPerBlock;
  rmsnorm_quant_long_kernel<<<dim3(static_cast<uint32_t>(blocks)), dim3(256), 0,
                              stream>>>(x, rows, k, ldx, gamma, eps, q, scale, y,
                                        ldy);
  return hipGetLastError();
}

}  // namespace fp8w8a8
