// Per-row FP8 (E4M3) quantization: per-token dynamic for activations,
// per-output-channel static for weights (MOSS-VL quantization README,
// "FP8-Dynamic" recipe; the same arithmetic on rows of X[M,K] or W[N,K]).
//
// One wavefront owns one row.  The row is read from HBM once, with 16-byte
// buffer loads (the descriptor clips the ragged tail), into registers; the magnitude maximum is reduced on the bf16 bit
// patterns (integer order equals value order for non-negative floats) and
// then across the wave; the scale amax/448 is one IEEE division; each
// element is divided by the scale (the IEEE quotient, with the reciprocal
// part hoisted out of the row: make_divisor), clamped to +-448 and converted
// with round-to-nearest-even by v_cvt_pk_fp8_f32; codes leave as 8-byte
// stores that are contiguous across the wave.  HBM traffic is the algorithmic
// 2 bytes in + 1 byte out per element + 4 bytes of scale per row.
#include "device_common.h"
#include "launch.h"

namespace fp8w8a8 {

namespace detail {

constexpr int kRowsPerBlock = 4;  // 4 waves, one row each

template <int NV>
__global__ __launch_bounds__(256) void quant_rows_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int k, int64_t ld,
    uint8_t* __restrict__ q, float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock +
                      __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (row >= rows) return;
  const auto src = row_rsrc(x + row * ld, static_cast<uint32_t>(k) * 2u);
  uint4 v[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) v[i] = buf_load16_stream(src, (i * 64 + lane) * 16u);
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    m = pk_max_u16(m, bf16x2_abs_bits(v[i].x));
    m = pk_max_u16(m, bf16x2_abs_bits(v[i].y));
    m = pk_max_u16(m, bf16x2_abs_bits(v[i].z));
    m = pk_max_u16(m, bf16x2_abs_bits(v[i].w));
  }
  const uint32_t mrow = wave_max_u32(max(m & 0xffffu, m >> 16));
  const float s = row_scale(__uint_as_float(mrow << 16));
  const auto dst = row_rsrc(q + row * static_cast<int64_t>(k), static_cast<uint32_t>(k));
  quantize_row<NV>(v, make_divisor(s), [&](int i, uint2 c) {
    buf_store8(c, dst, (i * 64 + lane) * 8u);
  });
  if (lane == 0) scale[row] = s;
}

// Rows longer than the register-resident variants: two passes, the second
// re-reads the row (from L2 for rows of this size).
__global__ __launch_bounds__(256) void quant_rows_long_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t k, int64_t ld,
    uint8_t* __restrict__ q, float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const int64_t row =
      static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;
  const uint4* src = reinterpret_cast<const uint4*>(x + row * ld);
  const int64_t nvec = k >> 3;
  uint32_t m = 0;
  for (int64_t idx = lane; idx < nvec; idx += 64) {
    const uint4 v = src[idx];
    m = pk_max_u16(m, bf16x2_abs_bits(v.x));
    m = pk_max_u16(m, bf16x2_abs_bits(v.y));
    m = pk_max_u16(m, bf16x2_abs_bits(v.z));
    m = pk_max_u16(m, bf16x2_abs_bits(v.w));
  }
  const uint32_t mrow = wave_max_u32(max(m & 0xffffu, m >> 16));
  const float s = row_scale(__uint_as_float(mrow << 16));
  const RowDivisor d = make_divisor(s);
  uint2* dst = reinterpret_cast<uint2*>(q + row * k);
  for (int64_t idx = lane; idx < nvec; idx += 64) dst[idx] = quantize8(src[idx], d);
  if (lane == 0) scale[row] = s;
}

__global__ __launch_bounds__(256) void zero_fill_kernel(uint4* p, size_t n16) {
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
       i < n16; i += stride)
    p[i] = make_uint4(0, 0, 0, 0);
}

template <int NV>
hipError_t launch_nv(const uint16_t* x, int64_t rows, int64_t k, int64_t ld,
                     uint8_t* q, float* scale, hipStream_t stream) {
  const int64_t blocks = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  quant_rows_kernel<NV><<<dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, stream>>>(
        x, rows, static_cast<int>(k), ld, q, scale);
  return hipGetLastError();
}

}  // namespace detail
using namespace detail;

hipError_t launch_quant_rows(const uint16_t* x, int64_t rows, int64_t k,
                             int64_t ld, uint8_t* q, float* scale,
                             hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const int64_t nvec = k / 8;
  const int64_t per_lane = (nvec + 63) / 64;
  if (per_lane <= 1) return launch_nv<1>(x, rows, k, ld, q, scale, stream);
  if (per_lane <= 2) return launch_nv<2>(x, rows, k, ld, q, scale, stream);
  if (per_lane <= 4) return launch_nv<4>(x, rows, k, ld, q, scale, stream);
  if (per_lane <= 8) return launch_nv<8>(x, rows, k, ld, q, scale, stream);
  if (per_lane <= 12) return launch_nv<12>(x, rows, k, ld, q, scale, stream);
  if (per_lane <= 16) return launch_nv<16>(x, rows, k, ld, q, scale, stream);
  if (per_lane <= 24) return launch_nv<24>(x, rows, k, ld, q, scale, stream);
  const int64_t blocks = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  quant_rows_long_kernel<<<dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, stream>>>(
        x, rows, k, ld, q, scale);
  return hipGetLastError();
}

hipError_t launch_zero_fill(void* p, size_t bytes, hipStream_t stream) {
  if (bytes == 0) return hipSuccess;
  const size_t n16 = bytes / 16;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  zero_fill_kernel<<<dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, stream>>>(
        static_cast<uint4*>(p), n16);
  return hipGetLastError();
}

}  // namespace fp8w8a8
