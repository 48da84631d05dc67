// Measured peaks of the two roofs the Linear runs under, for reporting
// beside the published ones: the dense FP8 MFMA rate of a loop that does
// nothing but v_mfma_f32_32x32x64_f8f6f4 on register operands, with the
// shader clock it ran at, and the HBM read rate of a persistent streaming
// read.
// Benchmark tooling only: none of the method's arithmetic is here.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "fp8w8a8_peaks.h"

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kChains = 8;          // independent accumulators per wave
constexpr int kThreads = 256;

// Every wave issues kChains * iters MFMAs (131072 flop each) on operands
// that stay in registers; the accumulators are stored at the end so that
// nothing is dead.  Wave 0 of workgroup 0 also reads the shader-clock and
// the constant 100 MHz counters at its start and end.
__global__ __launch_bounds__(kThreads) void mfma_loop_kernel(
    float* __restrict__ out, unsigned long long* __restrict__ clk, int iters) {
  const bool timer = blockIdx.x == 0 && threadIdx.x < 64;
  unsigned long long c0 = 0, r0 = 0;
  if (timer) {
    c0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  // Codes 0x30..0x37 and 0x28..0x2f: small normal E4M3 values, so the
  // accumulators stay finite over any loop length used here.
  const int lane = threadIdx.x & 63;
  v8i a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = static_cast<int>(0x30303030u + 0x01010101u * ((lane + i) & 7));
    b[i] = static_cast<int>(0x28282828u + 0x01010101u * ((lane * 3 + i) & 7));
  }
  v16f acc[kChains];
  for (int j = 0; j < kChains; ++j)
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kChains; ++j)
      acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[j], 0, 0, 0,
                                                               0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < kChains; ++j)
    for (int e = 0; e < 16; ++e) s += acc[j][e];
  out[static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x] = s;
  if (timer) {
    const unsigned long long c1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    if (lane == 0) {
      clk[0] = c1 - c0;
      clk[1] = r1 - r0;
    }
  }
}

// A persistent read: kReadWorkgroups workgroups (4 per compute unit) step
// over the buffer, each round reading kUnroll 16-byte vectors per thread,
// all issued before any is used, with the nontemporal hint (the data is
// read once).  The XOR of what a thread read is stored, so nothing is dead.
constexpr int kUnroll = 8;
constexpr int64_t kReadWorkgroups = 1024;

typedef unsigned int v4u_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void read_stream_kernel(
    const v4u_t* __restrict__ src, int64_t n16, uint32_t* __restrict__ out) {
  uint32_t x = 0;
  const int64_t step = static_cast<int64_t>(gridDim.x) * kThreads * kUnroll;
  for (int64_t base = static_cast<int64_t>(blockIdx.x) * kThreads * kUnroll + threadIdx.x;
       base < n16; base += step) {
    v4u_t v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = base + u * kThreads;
      v[u] = i < n16 ? __builtin_nontemporal_load(src + i) : v4u_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  out[static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x] = x;
}

}  // namespace

extern "C" {

int64_t fp8w8a8_peaks_mfma_out_floats(int64_t workgroups) {
  return workgroups * kThreads;
}

int fp8w8a8_peaks_mfma_loop(float* out, unsigned long long* clk, int64_t workgroups,
                            int iters, void* stream) {
  if (!out || !clk) return 1;
  if (workgroups < 1 || workgroups > (int64_t{1} << 20) || iters < 1) return 2;
  mfma_loop_kernel<<<dim3(static_cast<uint32_t>(workgroups)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream)>>>(out, clk, iters);
  return hipGetLastError() == hipSuccess ? 0 : 7;
}

int64_t fp8w8a8_peaks_mfma_flops(int64_t workgroups, int iters) {
  return workgroups * (kThreads / 64) * kChains * static_cast<int64_t>(iters) *
         (2 * 32 * 32 * 64);
}

int64_t fp8w8a8_peaks_read_workgroups(int64_t bytes) {
  (void)bytes;
  return kReadWorkgroups;
}

int fp8w8a8_peaks_read_stream(const void* src, int64_t bytes, uint32_t* out,
                              void* stream) {
  if (!src || !out) return 1;
  if (bytes < 16 || bytes % 16 != 0) return 2;
  if (reinterpret_cast<uintptr_t>(src) % 16 != 0) return 3;
  read_stream_kernel<<<dim3(static_cast<uint32_t>(kReadWorkgroups)), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream)>>>(
      static_cast<const v4u_t*>(src), bytes / 16, out);
  return hipGetLastError() == hipSuccess ? 0 : 7;
}

}  // extern "C"
