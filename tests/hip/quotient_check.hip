// Test helper (not part of the library): exhaustive comparison of the
// quantizer's fast-path division with its general path.
//
// For every bf16 amax whose scale s = fl32(amax / 448) takes the fast path
// and every finite bf16 value v with |v| <= amax (signs alternating), the
// codes quantize8 produces on the fast path (reciprocal, one residual
// correction, no clamp, sign bits inserted afterwards) must equal the codes
// it produces on its general path (IEEE float32 quotient v / s, clamp to
// +-448, round to nearest even).  Those are all the (v, scale) pairs the fast
// path can meet, since every quantized row is bf16 and is divided by the
// scale of its own amax.
#include <hip/hip_runtime.h>

#include "../../fp8_w8a8_dynamic_amd/csrc/device_common.h"

namespace {

using namespace fp8w8a8;

constexpr int kExpLo = -53, kExpHi = 69;  // covers every fast-path scale

__global__ __launch_bounds__(256) void quotient_check_kernel(
    unsigned long long* cnt) {
  const uint32_t mant = blockIdx.x & 127u;
  const int e = kExpLo + static_cast<int>(blockIdx.x >> 7);
  const uint32_t amax_bits = static_cast<uint32_t>(e + 127) << 7 | mant;
  const RowDivisor fast = make_divisor(row_scale(__uint_as_float(amax_bits << 16)));
  if (!fast.fast) {
    if (threadIdx.x == 0) atomicAdd(&cnt[2], 1ull);
    return;
  }
  RowDivisor general = fast;
  general.fast = false;
  unsigned long long pairs = 0, bad = 0;
  for (uint32_t g0 = threadIdx.x * 8u; g0 <= amax_bits; g0 += blockDim.x * 8u) {
    uint32_t h[8];
#pragma unroll
    for (uint32_t i = 0; i < 8; ++i) {
      const uint32_t b = g0 + i;
      const bool in = b <= amax_bits;
      pairs += in;
      h[i] = (in ? b : 0u) | (((i ^ (g0 >> 3)) & 1u) << 15);
    }
    const uint4 v = make_uint4(h[0] | h[1] << 16, h[2] | h[3] << 16,
                               h[4] | h[5] << 16, h[6] | h[7] << 16);
    const uint2 a = quantize8(v, fast), c = quantize8(v, general);
    bad += (a.x != c.x) + (a.y != c.y);
  }
  atomicAdd(&cnt[0], pairs);
  if (bad) atomicAdd(&cnt[1], bad);
}

}  // namespace

// counts[0] = pairs checked, counts[1] = 8-code groups that differ,
// counts[2] = amax values skipped (scale off the fast path).  Returns the
// hipError_t of the first failing call (0 on success).
extern "C" int fp8w8a8_test_quotient_check(unsigned long long* counts) {
  unsigned long long* d = nullptr;
  hipError_t e = hipMalloc(&d, 3 * sizeof(unsigned long long));
  if (e != hipSuccess) return static_cast<int>(e);
  e = hipMemset(d, 0, 3 * sizeof(unsigned long long));
  if (e == hipSuccess) {
    const uint32_t blocks = static_cast<uint32_t>(kExpHi - kExpLo + 1) * 128u;
    quotient_check_kernel<<<dim3(blocks), dim3(256)>>>(d);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e == hipSuccess)
    e = hipMemcpy(counts, d, 3 * sizeof(unsigned long long), hipMemcpyDeviceToHost);
  const hipError_t f = hipFree(d);
  return static_cast<int>(e != hipSuccess ? e : f);
}
