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
//   1. ss = sum x^2 in float32 in the fixed block order of row_ops.h (per
//      512-value block a v_dot2 chain per lane and a DPP tree; blocks added
//      in order, across the row's waves through LDS), so every layout, and
//      the decode GEMV's staging, gives the same sum; a row whose
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
#include <cstdlib>

#include "device_common.h"
#include "launch.h"
#include "row_ops.h"

namespace fp8w8a8 {

namespace detail {

constexpr int kNormRowsPerBlock = 4;  // one-wave-per-row layouts

// Sum (SUM) or max (!SUM, non-negative floats) of one value per wave over
// the S waves that share a row; `slot` is this exchange's own LDS array.
// Every wave of the workgroup calls it (the barrier is unconditional).
template <int S, bool SUM>
__device__ __forceinline__ float row_combine(float v, float* slot, int wave) {
  if (S == 1) return v;
  if ((threadIdx.x & 63) == 0) slot[wave] = v;
  __syncthreads();
  const int first = (wave / S) * S;
  float r = slot[first];
#pragma unroll
  for (int j = 1; j < S; ++j)
    r = SUM ? r + slot[first + j] : __builtin_fmaxf(r, slot[first + j]);
  return r;
}

// The row's sum of squares in block order: this wave holds blocks
// part * NV .. part * NV + NV - 1 (vector i of a lane is in block
// part * NV + i); with S > 1 the block sums meet in LDS (blk: this row's
// S * NV slots) and every wave adds all of them in order.  Unconditional
// barrier for S > 1.
template <int NV, int S, bool SCALED>
__device__ __forceinline__ float row_sumsq(const uint4 (&v)[NV], float p,
                                           float* blk, int part) {
  float b[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i)
    b[i] = SCALED ? block_sumsq_scaled(v[i], p) : block_sumsq(v[i]);
  if (S == 1) {
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < NV; ++i) ss += b[i];
    return ss;
  }
  if ((threadIdx.x & 63) == 0) {
#pragma unroll
    for (int i = 0; i < NV; ++i) blk[part * NV + i] = b[i];
  }
  __syncthreads();
  float ss = 0.0f;
#pragma unroll
  for (int j = 0; j < S * NV; ++j) ss += blk[j];
  return ss;
}

// A row of k elements is split over S waves of a workgroup (4 / S rows per
// workgroup), each wave holding NV 16-byte vectors of the row per lane.
template <int NV, int S>
__global__ __launch_bounds__(256) void rmsnorm_quant_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int k, int64_t ldx,
    const uint16_t* __restrict__ gamma, float eps, uint8_t* __restrict__ q,
    float* __restrict__ scale, uint16_t* __restrict__ y, int64_t ldy) {
  __shared__ float s_blk[4][S * NV], s_blk2[4][S * NV], s_amx[4], s_amy[4];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rloc = wave / S;                     // row within the workgroup
  const int64_t row = static_cast<int64_t>(blockIdx.x) * (4 / S) + rloc;
  const int part = wave % S;
  // Waves past the last row still take part in the exchanges, with empty
  // descriptors (no memory is touched).
  const bool live = row < rows;
  const int64_t r = live ? row : 0;
  const uint32_t row_bytes = live ? static_cast<uint32_t>(k) * 2u : 0u;
  const auto src = row_rsrc(x + r * ldx, row_bytes);
  const auto gsrc = row_rsrc(gamma, row_bytes);
  const uint32_t v0 = static_cast<uint32_t>(part * NV * 64 + lane);
  uint4 v[NV], g[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) v[i] = buf_load16_stream(src, (v0 + i * 64) * 16u);
#pragma unroll
  for (int i = 0; i < NV; ++i) g[i] = buf_load16(gsrc, (v0 + i * 64) * 16u);
  float ss = row_sumsq<NV, S, false>(v, 1.0f, s_blk[rloc], part);
  float p = 1.0f;
  const bool rare = !sumsq_in_range(ss);   // uniform over the row's waves
  if (S == 1) {
    if (rare) {
      uint32_t m = 0;
#pragma unroll
      for (int i = 0; i < NV; ++i) m = amax8_bits(v[i], m);
      p = pow2_for_amax(wave_max_u32(max(m & 0xffffu, m >> 16)));
      ss = row_sumsq<NV, 1, true>(v, p, nullptr, 0);
    }
  } else {
    // The rare path's exchanges run for every row (their barriers must be
    // reached by all waves); only rows that need them use the results.
    uint32_t m = 0;
    if (rare) {
#pragma unroll
      for (int i = 0; i < NV; ++i) m = amax8_bits(v[i], m);
    }
    const float amx = row_combine<S, false>(
        __uint_as_float(wave_max_u32(max(m & 0xffffu, m >> 16)) << 16), s_amx, wave);
    if (rare) p = pow2_for_amax(__float_as_uint(amx) >> 16);
    const float ss2 = row_sumsq<NV, S, true>(v, p, s_blk2[rloc], part);
    if (rare) ss = ss2;
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
  am = row_combine<S, false>(__uint_as_float(wave_max_u32(__float_as_uint(am))),
                             s_amy, wave);
  const float s = scale_from_row_max(am);
  const auto dst = row_rsrc(q + r * static_cast<int64_t>(k),
                            live ? static_cast<uint32_t>(k) : 0u);
  quantize_row<NV>(v, make_divisor(s), [&](int i, uint2 c) {
    buf_store8(c, dst, (v0 + i * 64) * 8u);
  });
  if (y != nullptr) {
    const auto ydst = row_rsrc(y + r * ldy, row_bytes);
#pragma unroll
    for (int i = 0; i < NV; ++i) buf_store16(v[i], ydst, (v0 + i * 64) * 16u);
  }
  if (live && part == 0 && lane == 0) scale[row] = s;
}

// Rows longer than the register-resident variants: the same arithmetic,
// block by block, in three passes over the row (sum of squares, amax of y,
// output; a fourth for the amax of x on the rare, rescaled path), the later
// ones reading the row again from L2.  (x * 1) * (p f) is the same product
// as x * (p f).
__global__ __launch_bounds__(256) void rmsnorm_quant_long_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t k, int64_t ldx,
    const uint16_t* __restrict__ gamma, float eps, uint8_t* __restrict__ q,
    float* __restrict__ scale, uint16_t* __restrict__ y, int64_t ldy) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kNormRowsPerBlock +
                      __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (row >= rows) return;
  const uint4* src = reinterpret_cast<const uint4*>(x + row * ldx);
  const uint4* gsrc = reinterpret_cast<const uint4*>(gamma);
  const int64_t nvec = k >> 3;
  auto xv = [&](int64_t idx) { return idx < nvec ? src[idx] : make_uint4(0, 0, 0, 0); };
  auto gv = [&](int64_t idx) { return idx < nvec ? gsrc[idx] : make_uint4(0, 0, 0, 0); };
  float ss = 0.0f;
  for (int64_t base = 0; base < nvec; base += 64) ss += block_sumsq(xv(base + lane));
  float p = 1.0f;
  if (!sumsq_in_range(ss)) {
    uint32_t m = 0;
    for (int64_t base = 0; base < nvec; base += 64) m = amax8_bits(xv(base + lane), m);
    p = pow2_for_amax(wave_max_u32(max(m & 0xffffu, m >> 16)));
    ss = 0.0f;
    for (int64_t base = 0; base < nvec; base += 64)
      ss += block_sumsq_scaled(xv(base + lane), p);
  }
  const NormFactor nf = make_norm_factor(ss, k, eps, p);
  const float pa = nf.one_mul ? 1.0f : nf.p, fa = nf.one_mul ? nf.pf : nf.f;
  float am = 0.0f;
  for (int64_t base = 0; base < nvec; base += 64)
    norm8<false>(xv(base + lane), gv(base + lane), pa, fa, am);
  const float s = scale_from_row_max(__uint_as_float(wave_max_u32(__float_as_uint(am))));
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

template <int NV, int S>
hipError_t launch_norm_nv(const uint16_t* x, int64_t rows, int64_t k,
                          int64_t ldx, const uint16_t* gamma, float eps,
                          uint8_t* q, float* scale, uint16_t* y, int64_t ldy,
                          hipStream_t stream) {
  constexpr int kRows = 4 / S;
  const int64_t blocks = (rows + kRows - 1) / kRows;
  rmsnorm_quant_kernel<NV, S><<<dim3(static_cast<uint32_t>(blocks)), dim3(256),
                                0, stream>>>(x, rows, static_cast<int>(k), ldx,
                                             gamma, eps, q, scale, y, ldy);
  return hipGetLastError();
}

}  // namespace detail
using namespace detail;

// Waves per row: with the test hooks on, FP8W8A8_NORM_SPLIT=1|2|4 overrides
// the choice (tuning and tests); rows up to 4 x 12 vectors per lane take the
// register kernels.
int norm_split(int64_t rows, int64_t per_lane) {
  if (const char* e = test_hook("FP8W8A8_NORM_SPLIT")) {
    const int v = std::atoi(e);
    if (v == 1 || v == 2 || v == 4) return v;
  }
  // Measured at k = 4096 on MI355X: one wave per row is fastest once there
  // are thousands of rows (12.0 us at 4096 rows against 13.4 us split over
  // four), four waves per row when rows are few (2.8 us against 3.8 us for
  // one row, 3.2 against 3.8 for 64).
  if (per_lane < 4) return 1;
  return rows >= 2048 ? 1 : (rows >= 512 ? 2 : 4);
}

hipError_t launch_rmsnorm_quant(const uint16_t* x, int64_t rows, int64_t k,
                                int64_t ldx, const uint16_t* gamma, float eps,
                                uint8_t* q, float* scale, uint16_t* y,
                                int64_t ldy, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const int64_t per_lane = (k / 8 + 63) / 64;   // vectors per lane, one wave
  const int split = norm_split(rows, per_lane);
  const int64_t pw = (per_lane + split - 1) / split;   // per wave
#define FP8W8A8_NORM(NV, S) \
  return launch_norm_nv<NV, S>(x, rows, k, ldx, gamma, eps, q, scale, y, ldy, stream)
  if (split == 1) {
    if (pw <= 1) FP8W8A8_NORM(1, 1);
    if (pw <= 2) FP8W8A8_NORM(2, 1);
    if (pw <= 4) FP8W8A8_NORM(4, 1);
    if (pw <= 8) FP8W8A8_NORM(8, 1);
    if (pw <= 12) FP8W8A8_NORM(12, 1);
  } else if (split == 2) {
    if (pw <= 1) FP8W8A8_NORM(1, 2);
    if (pw <= 2) FP8W8A8_NORM(2, 2);
    if (pw <= 4) FP8W8A8_NORM(4, 2);
    if (pw <= 8) FP8W8A8_NORM(8, 2);
    if (pw <= 12) FP8W8A8_NORM(12, 2);
  } else {
    if (pw <= 1) FP8W8A8_NORM(1, 4);
    if (pw <= 2) FP8W8A8_NORM(2, 4);
    if (pw <= 4) FP8W8A8_NORM(4, 4);
    if (pw <= 8) FP8W8A8_NORM(8, 4);
    if (pw <= 12) FP8W8A8_NORM(12, 4);
  }
#undef FP8W8A8_NORM
  const int64_t blocks = (rows + kNormRowsPerBlock - 1) / kNormRowsPerBlock;
  rmsnorm_quant_long_kernel<<<dim3(static_cast<uint32_t>(blocks)), dim3(256), 0,
                              stream>>>(x, rows, k, ldx, gamma, eps, q, scale, y,
                                        ldy);
  return hipGetLastError();
}

}  // namespace fp8w8a8
