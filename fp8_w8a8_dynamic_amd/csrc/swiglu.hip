// SiLU-gated activation fused with the per-token FP8 quantization of its
// output, the input of down_proj.
//
// gate_proj and up_proj (packed as gate_up_proj) and down_proj are
// FP8_DYNAMIC Linears, so down_proj quantizes its input per token at run
// time (MOSS-VL quantization README, "FP8-Dynamic", and its packed-module
// mapping); the activation between them is not quantized
// (MOSS-VL-Realtime-FP8 article, component / precision map).  The pages do
// not name the activation: it is read as the gated SiLU of the language
// model's MLP, rounded as a BF16 module rounds it:
//     s = bf16(silu(g)),  silu(g) = g / (1 + exp(-g));   h = bf16(s * u)
// (s * u is exact in float32, so h is rounded once).  One kernel reads gate
// and up once, forms h in registers, takes the row's amax and writes the
// codes and the scale; h itself is written only on request.
//
// silu in float32 (row_ops.h): g * rcp(1 + 2^(-g log2 e)) for g >= -44
// (relative error about |g| 2^-24 from the rounding of the exponent plus a
// few ulps), an exponent-shifted g e^g below.  The choice is made per wave
// over its slice of the row, so the common case pays for one form; it
// changes no result.
//
// Layout: a row of i elements is split over S waves of a workgroup (S = 1,
// 2 or 4; 4 / S rows per workgroup of 4 waves), each wave holding NV
// 16-byte vectors (8 bf16) of gate and of up per lane; the S partial amax
// meet in LDS.  Loads and stores go through buffer descriptors that clip the
// ragged tail (padding lanes hold g = u = 0, hence h = 0).
#include "device_common.h"
#include "launch.h"
#include "row_ops.h"

namespace fp8w8a8 {

namespace detail {

template <int NV, int S>
__global__ __launch_bounds__(256) void swiglu_quant_kernel(
    const uint16_t* __restrict__ gate, int64_t ldg,
    const uint16_t* __restrict__ up, int64_t ldu, int64_t rows, int n,
    uint8_t* __restrict__ q, float* __restrict__ scale,
    uint16_t* __restrict__ h, int64_t ldh) {
  __shared__ float s_amax[4];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t row = static_cast<int64_t>(blockIdx.x) * (4 / S) + wave / S;
  const int part = wave % S;
  // Waves past the last row still take part in the LDS exchange; their
  // descriptors are empty, so they touch no memory.
  const bool live = row < rows;
  const int64_t r = live ? row : 0;
  const uint32_t row_bytes = live ? static_cast<uint32_t>(n) * 2u : 0u;
  const auto gsrc = row_rsrc(gate + r * ldg, row_bytes);
  const auto usrc = row_rsrc(up + r * ldu, row_bytes);
  const uint32_t v0 = static_cast<uint32_t>(part * NV * 64 + lane);
  uint4 g[NV], u[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) g[i] = buf_load16_stream(gsrc, (v0 + i * 64) * 16u);
#pragma unroll
  for (int i = 0; i < NV; ++i) u[i] = buf_load16_stream(usrc, (v0 + i * 64) * 16u);
  bool deep = false;
#pragma unroll
  for (int i = 0; i < NV; ++i) deep |= any_deep8(g[i]);
  float am = 0.0f;
  if (__builtin_amdgcn_ballot_w64(deep) == 0) {
#pragma unroll
    for (int i = 0; i < NV; ++i) g[i] = swiglu8<true>(g[i], u[i], am);
  } else {
#pragma unroll
    for (int i = 0; i < NV; ++i) g[i] = swiglu8<false>(g[i], u[i], am);
  }
  uint32_t m = wave_max_u32(__float_as_uint(am));  // non-negative floats
  if (S > 1) {
    if (lane == 0) s_amax[wave] = __uint_as_float(m);
    __syncthreads();
    const int first = (wave / S) * S;
#pragma unroll
    for (int j = 0; j < S; ++j) m = max(m, __float_as_uint(s_amax[first + j]));
  }
  // max |h| = bf16(max |s u|): the rounding is monotonic.
  const float s = row_scale(__uint_as_float(
      static_cast<uint32_t>(f32_to_bf16_bits(__uint_as_float(m))) << 16));
  const auto dst = row_rsrc(q + r * static_cast<int64_t>(n),
                            live ? static_cast<uint32_t>(n) : 0u);
  quantize_row<NV>(g, make_divisor(s), [&](int i, uint2 c) {
    buf_store8(c, dst, (v0 + i * 64) * 8u);
  });
  if (h != nullptr) {
    const auto hdst = row_rsrc(h + r * ldh, row_bytes);
#pragma unroll
    for (int i = 0; i < NV; ++i) buf_store16(g[i], hdst, (v0 + i * 64) * 16u);
  }
  if (live && part == 0 && lane == 0) scale[row] = s;
}

// Rows longer than 4 waves x 8 vectors per lane: one wave per row, two
// passes (amax, then the same h again, quantized), reading gate and up
// twice.  Each 8-vector chunk picks its silu form as the short kernels do.
__global__ __launch_bounds__(256) void swiglu_quant_long_kernel(
    const uint16_t* __restrict__ gate, int64_t ldg,
    const uint16_t* __restrict__ up, int64_t ldu, int64_t rows, int64_t n,
    uint8_t* __restrict__ q, float* __restrict__ scale,
    uint16_t* __restrict__ h, int64_t ldh) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 +
                      __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (row >= rows) return;
  const uint4* gs = reinterpret_cast<const uint4*>(gate + row * ldg);
  const uint4* us = reinterpret_cast<const uint4*>(up + row * ldu);
  const int64_t nvec = n >> 3;
  auto chunk = [&](int64_t idx, float& am) {
    const uint4 gv = idx < nvec ? gs[idx] : make_uint4(0, 0, 0, 0);
    const uint4 uv = idx < nvec ? us[idx] : make_uint4(0, 0, 0, 0);
    return __builtin_amdgcn_ballot_w64(any_deep8(gv)) == 0
               ? swiglu8<true>(gv, uv, am)
               : swiglu8<false>(gv, uv, am);
  };
  float am = 0.0f;
  for (int64_t base = 0; base < nvec; base += 64) chunk(base + lane, am);
  const uint32_t m = wave_max_u32(__float_as_uint(am));
  const float s = row_scale(__uint_as_float(
      static_cast<uint32_t>(f32_to_bf16_bits(__uint_as_float(m))) << 16));
  const RowDivisor d = make_divisor(s);
  uint2* dst = reinterpret_cast<uint2*>(q + row * n);
  uint4* hdst = h != nullptr ? reinterpret_cast<uint4*>(h + row * ldh) : nullptr;
  for (int64_t base = 0; base < nvec; base += 64) {
    float unused = 0.0f;
    const int64_t idx = base + lane;
    const uint4 hv = chunk(idx, unused);
    if (idx < nvec) {
      dst[idx] = quantize8(hv, d);
      if (hdst != nullptr) hdst[idx] = hv;
    }
  }
  if (lane == 0) scale[row] = s;
}

template <int NV, int S>
hipError_t launch_swiglu_nv(const uint16_t* gate, int64_t ldg,
                            const uint16_t* up, int64_t ldu, int64_t rows,
                            int64_t n, uint8_t* q, float* scale, uint16_t* h,
                            int64_t ldh, hipStream_t stream) {
  constexpr int kRowsPerBlock = 4 / S;
  const int64_t blocks = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  swiglu_quant_kernel<NV, S><<<dim3(static_cast<uint32_t>(blocks)), dim3(256),
                               0, stream>>>(gate, ldg, up, ldu, rows,
                                            static_cast<int>(n), q, scale, h, ldh);
  return hipGetLastError();
}

}  // namespace detail
using namespace detail;

hipError_t launch_swiglu_quant(const uint16_t* gate, int64_t ldg,
                               const uint16_t* up, int64_t ldu, int64_t rows,
                               int64_t n, uint8_t* q, float* scale,
                               uint16_t* h, int64_t ldh, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const int64_t per_lane = (n / 8 + 63) / 64;   // vectors per lane, one wave
#define FP8W8A8_SWIGLU(NV, S)                                                 \
  return launch_swiglu_nv<NV, S>(gate, ldg, up, ldu, rows, n, q, scale, h, ldh, \
                                 stream)
  if (per_lane <= 1) FP8W8A8_SWIGLU(1, 1);
  if (per_lane <= 2) FP8W8A8_SWIGLU(2, 1);
  if (per_lane <= 4) FP8W8A8_SWIGLU(4, 1);
  if (per_lane <= 8) FP8W8A8_SWIGLU(4, 2);
  if (per_lane <= 16) FP8W8A8_SWIGLU(4, 4);
  if (per_lane <= 24) FP8W8A8_SWIGLU(6, 4);
  if (per_lane <= 32) FP8W8A8_SWIGLU(8, 4);
#undef FP8W8A8_SWIGLU
  const int64_t blocks = (rows + 3) / 4;
  swiglu_quant_long_kernel<<<dim3(static_cast<uint32_t>(blocks)), dim3(256), 0,
                             stream>>>(gate, ldg, up, ldu, rows, n, q, scale, h,
                                       ldh);
  return hipGetLastError();
}

}  // namespace fp8w8a8
