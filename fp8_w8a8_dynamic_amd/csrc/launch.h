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

// RMSNorm of each row of x [rows, k] with weight gamma [k], then the
// per-row quantization of the bf16 result: codes [rows, k] contiguous, one
// float32 scale per row, and the bf16 result itself into y (row stride ldy)
// when y != nullptr.
hipError_t launch_rmsnorm_quant(const uint16_t* x, int64_t rows, int64_t k,
                                int64_t ldx, const uint16_t* gamma, float eps,
                                uint8_t* q, float* scale, uint16_t* y,
                                int64_t ldy, hipStream_t stream);

// h = bf16(bf16(silu(gate)) * up) over [rows, n], then the per-row
// quantization of h: codes [rows, n] contiguous, one float32 scale per row,
// and h itself into `h` (row stride ldh) when h != nullptr.
hipError_t launch_swiglu_quant(const uint16_t* gate, int64_t ldg,
                               const uint16_t* up, int64_t ldu, int64_t rows,
                               int64_t n, uint8_t* q, float* scale,
                               uint16_t* h, int64_t ldh, hipStream_t stream);

// FP8 KV-cache codec: rows of `width` values in groups of `group` (a power
// of two from 8 to 512 dividing width), one scale per group.
hipError_t launch_kv_quantize(const uint16_t* kv, int64_t rows, int64_t width,
                              int64_t ld, int64_t group, uint8_t* codes,
                              float* scales, hipStream_t stream);
hipError_t launch_kv_dequantize(const uint8_t* codes, const float* scales,
                                int64_t rows, int64_t width, int64_t group,
                                uint16_t* out, int64_t ldo, hipStream_t stream);
// INT8 group-wise cache: codes, one scale and one minimum per group; the
// read writes the dequantized history rows, then the bf16 tail rows.
hipError_t launch_kv_quantize_int8(const uint16_t* kv, int64_t rows,
                                   int64_t width, int64_t ld, int64_t group,
                                   uint8_t* codes, float* scales, float* mins,
                                   hipStream_t stream);
hipError_t launch_kv_read_int8(const uint8_t* codes, const float* scales,
                               const float* mins, int64_t hist,
                               const uint16_t* tail, int64_t tail_rows,
                               int64_t ldt, int64_t width, int64_t group,
                               uint16_t* out, int64_t ldo, hipStream_t stream);

// Prefill GEMM: y[m,n] = bf16(sum_k qx[m,k] qw[n,k] * sx[m] * sw[n]).
// The plan fixes the tile configuration and the number of K splits; with
// splits > 1 the GEMM writes float32 partial sums [splits, m, n] to `part`
// (gemm_partial_bytes) and a second kernel adds them in split order and
// applies the scales.
constexpr int kMaxSplits = 64;
struct GemmPlan {
  int cfg;
  int splits;
};
GemmPlan plan_gemm(int64_t m, int64_t n, int64_t k);
size_t gemm_partial_bytes(const GemmPlan& p, int64_t m, int64_t n);
hipError_t launch_gemm(const GemmPlan& p, const uint8_t* qx, const float* sx,
                       const uint8_t* qw, const float* sw, int64_t m, int64_t n,
                       int64_t k, uint16_t* y, int64_t ldy, float* part,
                       hipStream_t stream);

// Decode GEMV (m <= kGemvMaxM).  If x != nullptr the activations are
// quantized inside the kernel (fused; only where gemv_fused_fits), otherwise
// qx/sx are read.
constexpr int kGemvMaxM = 16;
bool gemv_fused_fits(int64_t m, int64_t n, int64_t k);
hipError_t launch_gemv(const uint16_t* x, int64_t ldx, const uint8_t* qx,
                       const float* sx, const uint8_t* qw, const float* sw,
                       int64_t m, int64_t n, int64_t k, uint16_t* y,
                       int64_t ldy, hipStream_t stream);

// Decode GEMV with a BF16 pre-step fused into its activation staging:
// kPreRmsNorm (x, gamma = x2, eps; needs k % 512 == 0) or kPreSwiGlu
// (gate = x, up = x2 with row stride ld2).  The codes are bit-identical to
// those of launch_rmsnorm_quant / launch_swiglu_quant.
constexpr int kPreRmsNorm = 1;
constexpr int kPreSwiGlu = 2;
bool gemv_pre_fits(int pre, int64_t m, int64_t n, int64_t k);
hipError_t launch_gemv_pre(int pre, const uint16_t* x, int64_t ldx,
                           const uint16_t* x2, int64_t ld2, float eps,
                           const uint8_t* qw, const float* sw, int64_t m,
                           int64_t n, int64_t k, uint16_t* y, int64_t ldy,
                           hipStream_t stream);

// Token-group GEMV, kGemvMaxM < m <= kGemvTokMaxM, on quantized activations.
constexpr int kGemvTokMaxM = 64;
hipError_t launch_gemv_tok(const uint8_t* qx, const float* sx,
                           const uint8_t* qw, const float* sw, int64_t m,
                           int64_t n, int64_t k, uint16_t* y, int64_t ldy,
                           hipStream_t stream);

hipError_t launch_zero_fill(void* p, size_t bytes, hipStream_t stream);

}  // namespace fp8w8a8
