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
#include <algorithm>
#include <cstdlib>

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

// Few rows (a decode or mid-size chunk of tokens): one wave per row gives
// too few waves to keep the memory system busy, so S waves share a row
// (a 4-wave workgroup holds 4 / S rows).  Wave w of a row holds the
// 16-byte vectors i * 64 S + 64 w + lane, i < NV; the waves' maxima meet in
// LDS; each element is then quantized with the same device functions as
// above, so codes and scale are those of quant_rows_kernel.
template <int NV, int S>
__global__ __launch_bounds__(256) void quant_rows_split_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int k, int64_t ld,
    uint8_t* __restrict__ q, float* __restrict__ scale) {
  static_assert(S == 2 || S == 4, "2 or 4 waves per row");
  __shared__ uint32_t wmax[4];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int part = wave % S;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * (4 / S) + wave / S;
  const bool live = row < rows;
  const int64_t r = live ? row : 0;
  const auto src = row_rsrc(x + r * ld, live ? static_cast<uint32_t>(k) * 2u : 0u);
  uint4 v[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i)
    v[i] = buf_load16_stream(src, ((i * S + part) * 64 + lane) * 16u);
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    m = pk_max_u16(m, bf16x2_abs_bits(v[i].x));
    m = pk_max_u16(m, bf16x2_abs_bits(v[i].y));
    m = pk_max_u16(m, bf16x2_abs_bits(v[i].z));
    m = pk_max_u16(m, bf16x2_abs_bits(v[i].w));
  }
  const uint32_t mw = wave_max_u32(max(m & 0xffffu, m >> 16));
  if (lane == 0) wmax[wave] = mw;
  __syncthreads();
  uint32_t mrow = 0;
#pragma unroll
  for (int j = 0; j < S; ++j) mrow = max(mrow, wmax[wave - part + j]);
  if (!live) return;
  const float s = row_scale(__uint_as_float(mrow << 16));
  const auto dst = row_rsrc(q + r * static_cast<int64_t>(k), static_cast<uint32_t>(k));
  quantize_row<NV>(v, make_divisor(s), [&](int i, uint2 c) {
    buf_store8(c, dst, ((i * S + part) * 64 + lane) * 8u);
  });
  if (lane == 0 && part == 0) scale[r] = s;
}

// Several matrices' rows in one launch (fp8w8a8_quantize_act_group): one
// row per workgroup, its four waves sharing it as in quant_rows_split_kernel
// (wave w holds the 16-byte vectors i * 256 + 64 w + lane, i < NV, NV sized
// for the longest row; vectors past a shorter row read as 0 through the
// descriptor and are never stored).  The workgroup finds its item by
// comparing its index with the items' first rows.  Codes and scales are
// those of quant_rows_kernel for every row.
struct QuantGroupArgs {
  QuantItem it[kGroupMax];
  int count;
};

template <int NV>
__global__ __launch_bounds__(256) void quant_group_kernel(const QuantGroupArgs a) {
  __shared__ uint32_t wmax[4];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t b = blockIdx.x;
  int i = 0;
  for (int j = 1; j < a.count; ++j)
    if (b >= a.it[j].row0) i = j;
  const QuantItem& it = a.it[i];
  const int64_t row = b - it.row0;
  const int k = static_cast<int>(it.k);
  const auto src = row_rsrc(it.x + row * it.ld, static_cast<uint32_t>(k) * 2u);
  uint4 v[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) v[j] = buf_load16_stream(src, ((j * 4 + wave) * 64 + lane) * 16u);
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    m = pk_max_u16(m, bf16x2_abs_bits(v[j].x));
    m = pk_max_u16(m, bf16x2_abs_bits(v[j].y));
    m = pk_max_u16(m, bf16x2_abs_bits(v[j].z));
    m = pk_max_u16(m, bf16x2_abs_bits(v[j].w));
  }
  const uint32_t mw = wave_max_u32(max(m & 0xffffu, m >> 16));
  if (lane == 0) wmax[wave] = mw;
  __syncthreads();
  const uint32_t mrow = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
  const float s = row_scale(__uint_as_float(mrow << 16));
  const auto dst = row_rsrc(it.q + row * it.k, static_cast<uint32_t>(k));
  quantize_row<NV>(v, make_divisor(s), [&](int j, uint2 c) {
    buf_store8(c, dst, ((j * 4 + wave) * 64 + lane) * 8u);
  });
  if (lane == 0 && wave == 0) it.scale[row] = s;
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

template <int NV, int S>
hipError_t launch_split(const uint16_t* x, int64_t rows, int64_t k, int64_t ld,
                        uint8_t* q, float* scale, hipStream_t stream) {
  const int64_t blocks = (rows + (4 / S) - 1) / (4 / S);
  quant_rows_split_kernel<NV, S><<<dim3(static_cast<uint32_t>(blocks)), dim3(256), 0,
                                   stream>>>(x, rows, static_cast<int>(k), ld, q, scale);
  return hipGetLastError();
}

// Waves per row for few rows.  With the test hooks on,
// FP8W8A8_QUANT_SPLIT=1|2|4 overrides (tuning and tests).
int quant_split(int64_t rows, int64_t per_lane) {
  int sp = rows < 512 ? 4 : rows < 2048 ? 2 : 1;
  if (const char* e = test_hook("FP8W8A8_QUANT_SPLIT")) {
    const int v = std::atoi(e);
    if (v == 1 || v == 2 || v == 4) sp = v;
  }
  if (per_lane < 2) sp = 1;
  return sp;
}

}  // namespace detail
using namespace detail;

hipError_t launch_quant_rows(const uint16_t* x, int64_t rows, int64_t k,
                             int64_t ld, uint8_t* q, float* scale,
                             hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const int64_t nvec = k / 8;
  const int64_t per_lane = (nvec + 63) / 64;
  const int sp = per_lane <= 24 ? quant_split(rows, per_lane) : 1;
  if (sp > 1) {
    const int64_t pl = (per_lane + sp - 1) / sp;   // vectors per lane
#define FP8W8A8_SPLIT(S)                                                  \
    if (pl <= 1) return launch_split<1, S>(x, rows, k, ld, q, scale, stream); \
    if (pl <= 2) return launch_split<2, S>(x, rows, k, ld, q, scale, stream); \
    if (pl <= 3) return launch_split<3, S>(x, rows, k, ld, q, scale, stream); \
    if (pl <= 4) return launch_split<4, S>(x, rows, k, ld, q, scale, stream); \
    if (pl <= 6) return launch_split<6, S>(x, rows, k, ld, q, scale, stream); \
    if (pl <= 8) return launch_split<8, S>(x, rows, k, ld, q, scale, stream); \
    return launch_split<12, S>(x, rows, k, ld, q, scale, stream);
    if (sp == 2) { FP8W8A8_SPLIT(2) }
    FP8W8A8_SPLIT(4)
#undef FP8W8A8_SPLIT
  }
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

hipError_t launch_quant_group(const QuantItem* items, int count, hipStream_t stream) {
  if (count < 1 || count > kGroupMax) return hipErrorInvalidValue;
  QuantGroupArgs a{};
  a.count = count;
  int64_t rows = 0, kmax = 0;
  for (int i = 0; i < count; ++i) {
    a.it[i] = items[i];
    a.it[i].row0 = rows;
    rows += items[i].rows;
    kmax = std::max(kmax, items[i].k);
  }
  if (rows == 0) return hipSuccess;
  if (rows > (int64_t{1} << 31) - 1 || kmax > kQuantGroupMaxK) return hipErrorInvalidValue;
  const dim3 grid(static_cast<uint32_t>(rows)), block(256);
  switch ((kmax + 2047) / 2048) {
    case 1: quant_group_kernel<1><<<grid, block, 0, stream>>>(a); break;
    case 2: quant_group_kernel<2><<<grid, block, 0, stream>>>(a); break;
    case 3: quant_group_kernel<3><<<grid, block, 0, stream>>>(a); break;
    case 4: quant_group_kernel<4><<<grid, block, 0, stream>>>(a); break;
    case 5: case 6: quant_group_kernel<6><<<grid, block, 0, stream>>>(a); break;
    default: quant_group_kernel<8><<<grid, block, 0, stream>>>(a); break;
  }
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
