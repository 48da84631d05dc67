// Device helpers shared by the FP8_DYNAMIC kernels (gfx950 only).
//
// E4M3 here is the OCP float8_e4m3fn format the MOSS-VL quantization README
// names for the FP8-Dynamic recipe: 4 exponent bits (bias 7), 3 mantissa
// bits, no infinities, largest finite magnitude 448.  gfx950 converts to and
// multiplies this exact format in hardware (v_cvt_pk_fp8_f32, the f8f6f4
// MFMA family with format selector 0), so no byte translation is needed
// anywhere on the path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8w8a8 {

constexpr float kE4M3Max = 448.0f;

// bfloat16 is the upper half of a float32: widening is a shift / mask.
__device__ __forceinline__ float bf16_lo(uint32_t w) {
  return __uint_as_float(w << 16);
}
__device__ __forceinline__ float bf16_hi(uint32_t w) {
  return __uint_as_float(w & 0xffff0000u);
}

// Magnitudes of two packed bf16 as 16-bit integers.  For non-negative
// floats the bit patterns order exactly like the values, so the row amax can
// be taken on integers (one packed max per two elements) and widened once.
__device__ __forceinline__ uint32_t bf16x2_abs_bits(uint32_t w) {
  return w & 0x7fff7fffu;
}
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  uint32_t lo = max(a & 0xffffu, b & 0xffffu);
  uint32_t hi = max(a >> 16, b >> 16);
  return lo | (hi << 16);
}
__device__ __forceinline__ float amax_bits_to_float(uint32_t packed) {
  uint32_t m = max(packed & 0xffffu, packed >> 16);
  return __uint_as_float(m << 16);
}

// Row scale: scale = amax / 448 with one IEEE float32 division (the default
// lowering of '/' for float on gfx950 is correctly rounded; the library is
// never built with fast-math).
__device__ __forceinline__ float row_scale(float amax) {
  return amax / kE4M3Max;
}

// fl32(v / scale); a zero scale means an all-zero row: keep v (a signed zero).
__device__ __forceinline__ float quotient(float v, float scale) {
  return v / scale;
}

// One row's divisor.  Every element of a row is divided by the same scale,
// so the reciprocal can be formed once per row: r = rcp(s) refined by one
// Newton step.  gfx950's correctly rounded division is that reciprocal,
// q0 = v*r, two residual corrections q += fma(-s, q, v)*r, with range
// scaling (v_div_scale / v_div_fmas) and a special-case pass (v_div_fixup)
// around it.  The fast path (2^-60 <= s <= 2^60, where the scaling is
// inactive) keeps one residual correction: its quotient can differ from the
// IEEE quotient by one ulp (it does for about 0.2 % of pairs), but its E4M3
// code never does for the values this quantizer divides.  Every row it
// quantizes is bfloat16 and its scale is fl32(amax / 448) of that row's own
// bf16 amax, so the fast path only ever sees pairs (v, amax) of finite bf16
// values with |v| <= amax: all 266,928,097 such pairs with a fast-path scale
// give the codes of the IEEE quotient on gfx950 (an exhaustive GPU test
// compares this path with the general one over all of them).  Other scales
// (zero, subnormal or extreme) take the plain IEEE division.
struct RowDivisor {
  float s, r;
  bool fast;
};

__device__ __forceinline__ RowDivisor make_divisor(float s) {
  RowDivisor d;
  d.s = s;
  const float r0 = __builtin_amdgcn_rcpf(s);
  d.r = __builtin_fmaf(__builtin_fmaf(-s, r0, 1.0f), r0, r0);
  d.fast = s >= 0x1p-60f && s <= 0x1p60f;
  return d;
}

// Quotient magnitude for a = |v| on the fast path (one residual
// correction; the sequence is odd in v, so the sign can be set afterwards).
__device__ __forceinline__ float quotient_mag(float a, const RowDivisor& d) {
  const float q0 = a * d.r;
  return __builtin_fmaf(__builtin_fmaf(-d.s, q0, a), d.r, q0);
}

// Four float32 quotients -> four E4M3 codes packed little-endian in a dword
// (code of `a` in the lowest byte).  The clamp to +-448 makes the hardware
// conversion's round-to-nearest-even saturate instead of overflowing.
__device__ __forceinline__ uint32_t encode4(float a, float b, float c,
                                            float d) {
  a = __builtin_amdgcn_fmed3f(a, -kE4M3Max, kE4M3Max);
  b = __builtin_amdgcn_fmed3f(b, -kE4M3Max, kE4M3Max);
  c = __builtin_amdgcn_fmed3f(c, -kE4M3Max, kE4M3Max);
  d = __builtin_amdgcn_fmed3f(d, -kE4M3Max, kE4M3Max);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return static_cast<uint32_t>(w);
}

// Four non-negative quotients that are below 464 (the E4M3 rounding boundary
// above 448) -> four codes without the clamp: round-to-nearest-even already
// lands on at most 448.  Every quotient of a row by that row's own scale is
// below 464: |v| <= amax and s = fl32(amax / 448) >= (amax / 448)(1 - 2^-24),
// so |v| / s <= 448 (1 + 2^-23), and the fast path's quotient is within one
// ulp of that.
__device__ __forceinline__ uint32_t encode4_mag(float a, float b, float c,
                                                float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return static_cast<uint32_t>(w);
}

// The sign bits of four bf16 packed in two dwords (element order lo(w0),
// hi(w0), lo(w1), hi(w1)) moved to bit 7 of bytes 0..3: v_perm_b32 picks
// byte 1 and byte 3 of each dword.
__device__ __forceinline__ uint32_t sign_bytes(uint32_t w0, uint32_t w1) {
  return __builtin_amdgcn_perm(w1, w0, 0x07050301u) & 0x80808080u;
}

// Quantize 8 bf16 (one 16-byte vector) of a row with that row's divisor ->
// 8 codes.  Fast path (d.fast): magnitudes are divided and the sign bits
// inserted afterwards (so -0 and negative values whose quotient underflows
// keep their sign, as the IEEE quotient's sign does).
__device__ __forceinline__ uint2 quantize8_fast(uint4 v, const RowDivisor& d) {
  uint2 out;
  out.x = encode4_mag(quotient_mag(__builtin_fabsf(bf16_lo(v.x)), d),
                      quotient_mag(__builtin_fabsf(bf16_hi(v.x)), d),
                      quotient_mag(__builtin_fabsf(bf16_lo(v.y)), d),
                      quotient_mag(__builtin_fabsf(bf16_hi(v.y)), d)) |
          sign_bytes(v.x, v.y);
  out.y = encode4_mag(quotient_mag(__builtin_fabsf(bf16_lo(v.z)), d),
                      quotient_mag(__builtin_fabsf(bf16_hi(v.z)), d),
                      quotient_mag(__builtin_fabsf(bf16_lo(v.w)), d),
                      quotient_mag(__builtin_fabsf(bf16_hi(v.w)), d)) |
          sign_bytes(v.z, v.w);
  return out;
}

// General path: the IEEE float32 quotient, clamped, for any scale; a zero
// scale (amax == 0: every element is +-0) gives the sign bits as codes.
__device__ __forceinline__ uint2 quantize8_general(uint4 v, const RowDivisor& d) {
  uint2 out;
  const float scale = d.s;
  if (scale == 0.0f) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t r[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      uint32_t a = w[2 * i], b = w[2 * i + 1];
      r[i] = ((a >> 15) & 1u) << 7 | ((a >> 31) & 1u) << 15 |
             ((b >> 15) & 1u) << 23 | ((b >> 31) & 1u) << 31;
    }
    out.x = r[0];
    out.y = r[1];
    return out;
  }
  out.x = encode4(quotient(bf16_lo(v.x), scale), quotient(bf16_hi(v.x), scale),
                  quotient(bf16_lo(v.y), scale), quotient(bf16_hi(v.y), scale));
  out.y = encode4(quotient(bf16_lo(v.z), scale), quotient(bf16_hi(v.z), scale),
                  quotient(bf16_lo(v.w), scale), quotient(bf16_hi(v.w), scale));
  return out;
}

__device__ __forceinline__ uint2 quantize8(uint4 v, const RowDivisor& d) {
  return d.fast ? quantize8_fast(v, d) : quantize8_general(v, d);
}

// A row's NV vectors (8 bf16 each) -> NV x 8 codes, with the fast/general
// choice made once for the row; store(i, codes) receives each vector's
// codes as soon as they are formed (keeps few of them live at once).
template <int NV, typename Store>
__device__ __forceinline__ void quantize_row(const uint4 (&v)[NV],
                                             const RowDivisor& d, Store store) {
  if (d.fast) {
#pragma unroll
    for (int i = 0; i < NV; ++i) store(i, quantize8_fast(v[i], d));
  } else {
#pragma unroll
    for (int i = 0; i < NV; ++i) store(i, quantize8_general(v[i], d));
  }
}

// Max over the 64 lanes of a wave (result valid in every lane), with DPP
// moves (no LDS round trips): quad, 8-lane, 16-lane (row) maxima, then the
// row broadcasts fold rows 0-2 into row 3, so lane 63 holds the maximum.
// Lanes a move does not write keep 0, the identity of an unsigned max.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(
      0, static_cast<int>(x), CTRL, ROW_MASK, 0xf, false));
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<0xb1, 0xf>(v));    // quad_perm [1,0,3,2]
  v = max(v, dpp_u32<0x4e, 0xf>(v));    // quad_perm [2,3,0,1]
  v = max(v, dpp_u32<0x141, 0xf>(v));   // row_half_mirror
  v = max(v, dpp_u32<0x140, 0xf>(v));   // row_mirror
  v = max(v, dpp_u32<0x142, 0xa>(v));   // row_bcast:15 into rows 1 and 3
  v = max(v, dpp_u32<0x143, 0xc>(v));   // row_bcast:31 into rows 2 and 3
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 63));
}

// float32 -> bfloat16 bits, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 h = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, h);
}

typedef float float2_vt __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_vt __attribute__((ext_vector_type(2)));

// Two float32 -> two bfloat16 (round to nearest even) packed in one dword,
// lo in the low half: one v_cvt_pk_bf16_f32 (two scalar conversions would be
// packed with extra shifts and ORs).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const float2_vt f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_vt));
}

// ---- global -> LDS copies (buffer_load_dwordx4 ... lds) -------------------

typedef int v4i_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

// s_waitcnt immediate for "at most n vector-memory operations outstanding"
// (gfx9 encoding; expcnt and lgkmcnt left at their maxima).
constexpr int vmcnt_imm(int n) {
  return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8);
}

// Buffer resource for `bytes` bytes at `base` (raw buffer, stride 0).  Loads
// at offsets >= bytes return zero.
__device__ __forceinline__ v4i_t make_rsrc(const uint8_t* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  v4i_t r;
  r[0] = static_cast<int>(static_cast<uint32_t>(a));
  r[1] = static_cast<int>(static_cast<uint32_t>(a >> 32) & 0xffffu);
  r[2] = static_cast<int>(bytes);
  r[3] = 0x00020000;  // raw 32-bit data format, no swizzle
  return r;
}

// Register loads and stores through a buffer resource covering one row:
// the range check is the descriptor's, so a row's ragged tail needs no
// branches (loads past the end return 0, stores past the end are dropped,
// neither touches memory), and straight-line code keeps the compiler's
// wait counts exact.  `base` must be wave-uniform.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* base,
                                                          uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0,
                                           static_cast<int>(bytes), 0x00020000);
}

typedef unsigned int v4u32_t __attribute__((ext_vector_type(4)));
typedef unsigned int v2u32_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r,
                                            uint32_t off) {
  const v4u32_t t = __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, 0);
  return make_uint4(t.x, t.y, t.z, t.w);
}

// Cache policy of the loads and stores of data that a call touches once
// (activation rows, codes and outputs of the row kernels, KV-cache rows,
// the GEMV's weights): the nontemporal bit (bit 1 of the policy operand,
// "nt" in the instruction).  Measured on MI355X with buffers rotated past
// the last-level cache, it raises the decode GEMVs' weight streaming by
// ~8 % and the KV-cache reads by 17-26 %, and costs the other row kernels
// nothing.
constexpr int kStreamPolicy = 2;

__device__ __forceinline__ uint4 buf_load16_stream(__amdgpu_buffer_rsrc_t r,
                                                   uint32_t off) {
  const v4u32_t t = __builtin_amdgcn_raw_buffer_load_b128(
      r, static_cast<int>(off), 0, kStreamPolicy);
  return make_uint4(t.x, t.y, t.z, t.w);
}

__device__ __forceinline__ uint4 load16_stream(const void* p) {
  const v4u32_t t = __builtin_nontemporal_load(static_cast<const v4u32_t*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}

__device__ __forceinline__ void buf_store8(uint2 v, __amdgpu_buffer_rsrc_t r,
                                           uint32_t off) {
  const v2u32_t t = {v.x, v.y};
  __builtin_amdgcn_raw_buffer_store_b64(t, r, static_cast<int>(off), 0,
                                        kStreamPolicy);
}

__device__ __forceinline__ void buf_store16(uint4 v, __amdgpu_buffer_rsrc_t r,
                                            uint32_t off) {
  const v4u32_t t = {v.x, v.y, v.z, v.w};
  __builtin_amdgcn_raw_buffer_store_b128(t, r, static_cast<int>(off), 0,
                                         kStreamPolicy);
}

// One 16-byte-per-lane copy global -> LDS: the wave's 64 x 16 bytes land
// contiguously at LDS byte address `lds` (M0, wave-uniform).  Inline asm so
// that the compiler's wait-count insertion leaves it alone; the instruction
// has no register result, and callers wait for it explicitly (vmcnt, then a
// barrier) before reading what it wrote.
__device__ __forceinline__ void lds_copy16(v4i_t rsrc, uint32_t voff,
                                           uint32_t soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(soff), "s"(lds)
               : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_t*)p));
}

}  // namespace fp8w8a8
