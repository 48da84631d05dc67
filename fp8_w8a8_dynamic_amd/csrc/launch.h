// Internal launchers behind the C ABI (not exported).  Every launcher
// assumes its arguments were validated by api.cpp and returns the
// hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fp8w8a8 {

// Per-row quantization of a bf16 matrix [rows, k] (row stride ld elements):
// codes [rows, k] contiguous and one float32 scale per row.
hipError_t launch_quant_rows(const uint16_t* x, int64_t rows, int64_t k,
                             int64_t ld, uint8_t* q, float* scale,
                             hipStream_t stream);

// Prefill GEMM: y[m,n] = bf16(sum_k qx[m,k] qw[n,k] * sx[m] * sw[n]).
hipError_t launch_gemm(const uint8_t* qx, const float* sx, const uint8_t* qw,
                       const float* sw, int64_t m, int64_t n, int64_t k,
                       uint16_t* y, int64_t ldy, hipStream_t stream);

// Decode GEMV (m <= kGemvMaxM).  If x != nullptr the activations are
// quantized inside the kernel (fused); otherwise qx/sx are read.
constexpr int kGemvMaxM = 16;
struct GemvPlan {
  int split_k;     // K slices per output tile, reduced in fixed order
  int k_chunk;     // bytes of K per workgroup (k / split_k)
};
GemvPlan plan_gemv(int64_t m, int64_t n, int64_t k, bool fused);
// Whether the fused decode kernel's LDS copy of the quantized chunk fits.
bool gemv_fused_fits(int64_t m, int64_t n, int64_t k);
// Bytes of float32 split-K partial tiles for one call (0 without split-K).
size_t gemv_partial_bytes(int64_t m, int64_t n, int64_t k, bool fused);
// Split-K arrival counters live in a fixed region at the start of every
// workspace (one per 16-channel tile), never used for anything else, so a
// workspace shared by calls of different shapes keeps them zero.
constexpr size_t kCounterBytes = 64 * 1024;
constexpr int64_t kMaxSplitTiles = kCounterBytes / 4;
hipError_t launch_gemv(const uint16_t* x, int64_t ldx, const uint8_t* qx,
                       const float* sx, const uint8_t* qw, const float* sw,
                       int64_t m, int64_t n, int64_t k, uint16_t* y,
                       int64_t ldy, unsigned* counters, float* partials,
                       hipStream_t stream);

hipError_t launch_zero_fill(void* p, size_t bytes, hipStream_t stream);

}  // namespace fp8w8a8
