// Key/value-cache codecs: FP8 E4M3 (below) and INT8 group-wise with a BF16
// residual window (further down).
//
// With the FP8 checkpoint under SGLang the KV cache uses the engine's own
// dtype, e.g. --kv-cache-dtype fp8_e4m3 (MOSS-VL quantization README, "KV
// cache").  The pages give only that dtype; the readings here: each token's
// K (or V) row is quantized with the activation quantizer's arithmetic, one
// dynamic float32 scale per group of `group` consecutive values (one KV head
// by default), and reading back gives bf16(fl32(dec(code) * scale)).
//
// Quantize: one wave per row (4 rows per workgroup), the row walked in
// chunks of 64 lanes x 8 values; a group (a power of two from 8 to 512
// values) is G / 8 consecutive lanes of one chunk, so its amax is a
// butterfly over those lanes, then every lane quantizes its 8 values with
// its group's divisor (the quantizer's device code, bit for bit).
// Read back: one wave per row, 8 codes per lane decoded exactly by
// v_cvt_pk_f32_fp8, one float32 multiply by the group's scale, one
// round-to-nearest-even to bf16.  Loads and stores go through per-row buffer
// descriptors, which clip the ragged last chunk.
#include "device_common.h"
#include "launch.h"

namespace fp8w8a8 {

namespace detail {

constexpr int kKvRowsPerBlock = 4;

// Max over aligned groups of L lanes (L a power of two, 1..64).
template <int L>
__device__ __forceinline__ uint32_t group_max_u32(uint32_t v) {
#pragma unroll
  for (int m = 1; m < L; m <<= 1)
    v = max(v, static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), m, 64)));
  return v;
}

template <int L>
__global__ __launch_bounds__(256) void kv_quant_kernel(
    const uint16_t* __restrict__ kv, int64_t rows, int width, int64_t ld,
    uint8_t* __restrict__ codes, float* __restrict__ scales) {
  constexpr int kGroup = L * 8;
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kKvRowsPerBlock +
                      __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (row >= rows) return;
  const int groups = width / kGroup;
  const auto src = row_rsrc(kv + row * ld, static_cast<uint32_t>(width) * 2u);
  const auto dst = row_rsrc(codes + row * static_cast<int64_t>(width),
                            static_cast<uint32_t>(width));
  float* srow = scales + row * static_cast<int64_t>(groups);
  for (int base = 0; base < width; base += 512) {
    const int v = base / 8 + lane;                 // this lane's vector
    const uint4 x = buf_load16_stream(src, static_cast<uint32_t>(v) * 16u);
    uint32_t m = pk_max_u16(pk_max_u16(bf16x2_abs_bits(x.x), bf16x2_abs_bits(x.y)),
                            pk_max_u16(bf16x2_abs_bits(x.z), bf16x2_abs_bits(x.w)));
    m = group_max_u32<L>(max(m & 0xffffu, m >> 16));
    const float s = row_scale(__uint_as_float(m << 16));
    buf_store8(quantize8(x, make_divisor(s)), dst, static_cast<uint32_t>(v) * 8u);
    const int gi = (v * 8) / kGroup;
    if ((lane & (L - 1)) == 0 && gi < groups) srow[gi] = s;
  }
}

typedef float float2_kv_t __attribute__((ext_vector_type(2)));

// 4 E4M3 codes (a dword, lowest byte first) times s -> 4 bf16 (2 dwords).
__device__ __forceinline__ uint2 dequant4(uint32_t c, float s) {
  const float2_kv_t lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(c), false);
  const float2_kv_t hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(c), true);
  return make_uint2(pack_bf16x2(lo.x * s, lo.y * s), pack_bf16x2(hi.x * s, hi.y * s));
}

template <int L>
__global__ __launch_bounds__(256) void kv_dequant_kernel(
    const uint8_t* __restrict__ codes, const float* __restrict__ scales,
    int64_t rows, int width, uint16_t* __restrict__ out, int64_t ldo) {
  constexpr int kGroup = L * 8;
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kKvRowsPerBlock +
                      __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (row >= rows) return;
  const int groups = width / kGroup;
  const auto csrc = row_rsrc(codes + row * static_cast<int64_t>(width),
                             static_cast<uint32_t>(width));
  const auto ssrc = row_rsrc(scales + row * static_cast<int64_t>(groups),
                             static_cast<uint32_t>(groups) * 4u);
  const auto dst = row_rsrc(out + row * ldo, static_cast<uint32_t>(width) * 2u);
  for (int base = 0; base < width; base += 512) {
    const int v = base / 8 + lane;
    const v2u32_t c = __builtin_amdgcn_raw_buffer_load_b64(
        csrc, static_cast<int>(v * 8), 0, 0);
    const float s = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
        ssrc, static_cast<int>(((v * 8) / kGroup) * 4), 0, 0));
    const uint2 a = dequant4(c.x, s), b = dequant4(c.y, s);
    buf_store16(make_uint4(a.x, a.y, b.x, b.y), dst, static_cast<uint32_t>(v) * 16u);
  }
}

// ---- INT8 group-wise cache with a BF16 residual window ---------------------
//
// The Transformers path of the checkpoint keeps the KV cache as HQQ INT8,
// groups of 64, with the newest 128 positions left in BF16; reading the cache
// dequantizes the history and appends that tail (MOSS-VL quantization README,
// "KV cache"; MOSS-VL-Realtime-FP8 article, KV-cache section).  HQQ's solver
// is not on the pages: the reading is its asymmetric min-max starting point,
// every step one IEEE float32 operation:
//   s = fl32(fl32(max - min) / 255)     (a zero max or min taken as +0)
//   q = clamp(rne(fl32(fl32(x - min) / s)), 0, 255)   (q = 0 when s = 0)
//   read back: bf16(fl32(fl32(q * s) + min))           (no fused multiply-add)

__device__ __forceinline__ float group_fmax(float v, int l) {
  for (int m = 1; m < l; m <<= 1) v = __builtin_fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}
__device__ __forceinline__ float group_fmin(float v, int l) {
  for (int m = 1; m < l; m <<= 1) v = __builtin_fminf(v, __shfl_xor(v, m, 64));
  return v;
}

// 4 values -> 4 uint8 codes in a dword (lowest byte first).
__device__ __forceinline__ uint32_t int8_codes4(float a, float b, float c, float d,
                                                float mn, float s) {
  const float v[4] = {a, b, c, d};
  uint32_t w = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float q = 0.0f;
    if (s > 0.0f) {
      q = __builtin_rintf((v[i] - mn) / s);
      q = __builtin_amdgcn_fmed3f(q, 0.0f, 255.0f);
    }
    w |= static_cast<uint32_t>(q) << (8 * i);   // exact: q is an integer in [0, 255]
  }
  return w;
}

template <int L>
__global__ __launch_bounds__(256) void kv_int8_quant_kernel(
    const uint16_t* __restrict__ kv, int64_t rows, int width, int64_t ld,
    uint8_t* __restrict__ codes, float* __restrict__ scales,
    float* __restrict__ mins) {
  constexpr int kGroup = L * 8;
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kKvRowsPerBlock +
                      __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (row >= rows) return;
  const int groups = width / kGroup;
  const auto src = row_rsrc(kv + row * ld, static_cast<uint32_t>(width) * 2u);
  const auto dst = row_rsrc(codes + row * static_cast<int64_t>(width),
                            static_cast<uint32_t>(width));
  float* srow = scales + row * static_cast<int64_t>(groups);
  float* mrow = mins + row * static_cast<int64_t>(groups);
  for (int base = 0; base < width; base += 512) {
    const int v = base / 8 + lane;
    const uint4 x = buf_load16_stream(src, static_cast<uint32_t>(v) * 16u);
    const float e[8] = {bf16_lo(x.x), bf16_hi(x.x), bf16_lo(x.y), bf16_hi(x.y),
                        bf16_lo(x.z), bf16_hi(x.z), bf16_lo(x.w), bf16_hi(x.w)};
    float lo = e[0], hi = e[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) {
      lo = __builtin_fminf(lo, e[i]);
      hi = __builtin_fmaxf(hi, e[i]);
    }
    // + 0 makes a zero extreme +0 (min/max of +0 and -0 may return either)
    lo = group_fmin(lo, L) + 0.0f;
    hi = group_fmax(hi, L) + 0.0f;
    const float s = (hi - lo) / 255.0f;
    buf_store8(make_uint2(int8_codes4(e[0], e[1], e[2], e[3], lo, s),
                          int8_codes4(e[4], e[5], e[6], e[7], lo, s)),
               dst, static_cast<uint32_t>(v) * 8u);
    const int gi = (v * 8) / kGroup;
    if ((lane & (L - 1)) == 0 && gi < groups) {
      srow[gi] = s;
      mrow[gi] = lo;
    }
  }
}

// 4 uint8 codes -> 4 bf16: fl32(fl32(q s) + mn), then round to bf16.
__device__ __forceinline__ uint2 int8_dequant4(uint32_t c, float s, float mn) {
#pragma clang fp contract(off)
  // (byte -> float is exact; it lowers to v_cvt_f32_ubyte0..3)
  const float a = static_cast<float>(c & 0xffu) * s + mn;
  const float b = static_cast<float>((c >> 8) & 0xffu) * s + mn;
  const float d = static_cast<float>((c >> 16) & 0xffu) * s + mn;
  const float e = static_cast<float>(c >> 24) * s + mn;
  return make_uint2(pack_bf16x2(a, b), pack_bf16x2(d, e));
}

// Output rows [0, hist) are the dequantized history, rows [hist, hist + tail)
// a copy of the bf16 residual window.
template <int L>
__global__ __launch_bounds__(256) void kv_int8_read_kernel(
    const uint8_t* __restrict__ codes, const float* __restrict__ scales,
    const float* __restrict__ mins, int64_t hist,
    const uint16_t* __restrict__ tail, int64_t tail_rows, int64_t ldt, int width,
    uint16_t* __restrict__ out, int64_t ldo) {
  constexpr int kGroup = L * 8;
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kKvRowsPerBlock +
                      __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (row >= hist + tail_rows) return;
  const auto dst = row_rsrc(out + row * ldo, static_cast<uint32_t>(width) * 2u);
  if (row >= hist) {
    const auto src = row_rsrc(tail + (row - hist) * ldt, static_cast<uint32_t>(width) * 2u);
    for (int base = 0; base < width; base += 512) {
      const uint32_t off = static_cast<uint32_t>(base / 8 + lane) * 16u;
      buf_store16(buf_load16_stream(src, off), dst, off);
    }
    return;
  }
  const int groups = width / kGroup;
  const auto csrc = row_rsrc(codes + row * static_cast<int64_t>(width),
                             static_cast<uint32_t>(width));
  const auto ssrc = row_rsrc(scales + row * static_cast<int64_t>(groups),
                             static_cast<uint32_t>(groups) * 4u);
  const auto msrc = row_rsrc(mins + row * static_cast<int64_t>(groups),
                             static_cast<uint32_t>(groups) * 4u);
  for (int base = 0; base < width; base += 512) {
    const int v = base / 8 + lane;
    const v2u32_t c = __builtin_amdgcn_raw_buffer_load_b64(csrc, v * 8, 0, 0);
    const int goff = ((v * 8) / kGroup) * 4;
    const float s = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(ssrc, goff, 0, 0));
    const float mn = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(msrc, goff, 0, 0));
    const uint2 a = int8_dequant4(c.x, s, mn), b = int8_dequant4(c.y, s, mn);
    buf_store16(make_uint4(a.x, a.y, b.x, b.y), dst, static_cast<uint32_t>(v) * 16u);
  }
}

}  // namespace detail
using namespace detail;

#define FP8W8A8_KV_GROUPS(X) X(1) X(2) X(4) X(8) X(16) X(32) X(64)

hipError_t launch_kv_quantize(const uint16_t* kv, int64_t rows, int64_t width,
                              int64_t ld, int64_t group, uint8_t* codes,
                              float* scales, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const dim3 grid(static_cast<uint32_t>((rows + kKvRowsPerBlock - 1) / kKvRowsPerBlock));
  const int w = static_cast<int>(width);
  switch (group / 8) {
#define FP8W8A8_KVQ(L)                                                          \
  case L:                                                                       \
    kv_quant_kernel<L><<<grid, dim3(256), 0, stream>>>(kv, rows, w, ld, codes, \
                                                       scales);                 \
    break;
    FP8W8A8_KV_GROUPS(FP8W8A8_KVQ)
#undef FP8W8A8_KVQ
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_kv_dequantize(const uint8_t* codes, const float* scales,
                                int64_t rows, int64_t width, int64_t group,
                                uint16_t* out, int64_t ldo, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const dim3 grid(static_cast<uint32_t>((rows + kKvRowsPerBlock - 1) / kKvRowsPerBlock));
  const int w = static_cast<int>(width);
  switch (group / 8) {
#define FP8W8A8_KVD(L)                                                           \
  case L:                                                                        \
    kv_dequant_kernel<L><<<grid, dim3(256), 0, stream>>>(codes, scales, rows, w, \
                                                         out, ldo);              \
    break;
    FP8W8A8_KV_GROUPS(FP8W8A8_KVD)
#undef FP8W8A8_KVD
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_kv_quantize_int8(const uint16_t* kv, int64_t rows,
                                   int64_t width, int64_t ld, int64_t group,
                                   uint8_t* codes, float* scales, float* mins,
                                   hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const dim3 grid(static_cast<uint32_t>((rows + kKvRowsPerBlock - 1) / kKvRowsPerBlock));
  const int w = static_cast<int>(width);
  switch (group / 8) {
#define FP8W8A8_KVQ8(L)                                                              \
  case L:                                                                            \
    kv_int8_quant_kernel<L><<<grid, dim3(256), 0, stream>>>(kv, rows, w, ld, codes, \
                                                            scales, mins);           \
    break;
    FP8W8A8_KV_GROUPS(FP8W8A8_KVQ8)
#undef FP8W8A8_KVQ8
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_kv_read_int8(const uint8_t* codes, const float* scales,
                               const float* mins, int64_t hist,
                               const uint16_t* tail, int64_t tail_rows,
                               int64_t ldt, int64_t width, int64_t group,
                               uint16_t* out, int64_t ldo, hipStream_t stream) {
  const int64_t rows = hist + tail_rows;
  if (rows == 0) return hipSuccess;
  const dim3 grid(static_cast<uint32_t>((rows + kKvRowsPerBlock - 1) / kKvRowsPerBlock));
  const int w = static_cast<int>(width);
  switch (group / 8) {
#define FP8W8A8_KVR8(L)                                                           \
  case L:                                                                         \
    kv_int8_read_kernel<L><<<grid, dim3(256), 0, stream>>>(                       \
        codes, scales, mins, hist, tail, tail_rows, ldt, w, out, ldo);            \
    break;
    FP8W8A8_KV_GROUPS(FP8W8A8_KVR8)
#undef FP8W8A8_KVR8
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

#undef FP8W8A8_KV_GROUPS

}  // namespace fp8w8a8
