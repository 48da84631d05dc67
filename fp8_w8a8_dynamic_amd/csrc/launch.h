// Internal launchers behind the C ABI (not exported).  Every launcher
// assumes its arguments were validated by api.cpp and returns the
// hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fp8w8a8 {

// Tuning and cross-check overrides (the kernel path, tile configuration,
// K splits, GEMV grouping, norm split) exist for the test suite only.  They
// are honoured only when the environment variable FP8W8A8_TEST_HOOKS is "1"
// the first time the library looks (read once per process); otherwise
// test_hook() returns nullptr for every name and no call ever reads the
// environment, so a stray variable cannot change a production kernel
// choice.  With the switch on, the named override is read at each call (the
// tests vary it between calls; workspace sizes must then be queried under
// the same overrides as the call).
const char* test_hook(const char* name);

// Per-row quantization of a bf16 matrix [rows, k] (row stride ld elements):
// codes [rows, k] contiguous and one float32 scale per row.
hipError_t launch_quant_rows(const uint16_t* x, int64_t rows, int64_t k,
                             int64_t ld, uint8_t* q, float* scale,
                             hipStream_t stream);

// Per-row quantization of up to kGroupMax bf16 matrices in one launch
// (codes and scales as launch_quant_rows gives for each); k <= kQuantGroupMaxK.
constexpr int kGroupMax = 16;
constexpr int64_t kQuantGroupMaxK = 16384;
struct QuantItem {
  const uint16_t* x;
  int64_t rows, k, ld;
  uint8_t* q;
  float* scale;
  int64_t row0;  // first row of the item in the launch (set by the launcher)
};
hipError_t launch_quant_group(const QuantItem* items, int count, hipStream_t stream);

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
// The GEMM with its bf16 output also quantized per token (codes q [m, n]
// contiguous, one float32 scale per row): the same y, q and scale as
// launch_gemm followed by launch_quant_rows on y.  Where the plan splits K
// and n <= kRequantMaxN, one kernel adds the splits, writes y and quantizes
// it (one launch and one read of y fewer).
constexpr int64_t kRequantMaxN = 16384;
hipError_t launch_gemm_requant(const GemmPlan& p, const uint8_t* qx, const float* sx,
                               const uint8_t* qw, const float* sw, int64_t m, int64_t n,
                               int64_t k, uint16_t* y, int64_t ldy, uint8_t* q,
                               float* scale, float* part, hipStream_t stream);

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

// Grouped one-token Linears (bf16 x [1, k] -> bf16 y [1, n] each, their
// quantization fused), up to kGroupMax of them in one launch; each item's
// output is bit-identical to launch_gemv on it alone.  k <= 12288.
struct GroupLinear {
  const uint16_t* x;
  const uint8_t* qw;
  const float* sw;
  uint16_t* y;
  int64_t n, k;
};
hipError_t launch_gemv_group_m1(const GroupLinear* items, int count,
                                hipStream_t stream);

// Grouped Linears on given codes (qx [m, k] E4M3 + sx [m] -> bf16 y [m, n]
// each, all items at the same m), 1 <= m <= kTokGroupMaxM, up to kGroupMax
// of them in one launch; qw in the MFMA-tile order of launch_tile_weights.
// n % 64 == 0, k % 128 == 0, k <= kTokGroupMaxK.
constexpr int kTokGroupMaxM = 256;
constexpr int kTokGroupMaxK = 16384;
struct TokLinear {
  const uint8_t* qx;
  const float* sx;
  const uint8_t* qw;
  const float* sw;
  uint16_t* y;
  int64_t n, k;
};
hipError_t launch_tok_group(const TokLinear* items, int count, int64_t m,
                            hipStream_t stream);
// The same launch with item rq's K summed in `splits` ranges (units of
// their own in the launch; raw float32 sums [splits, m, n] to `part`), then
// one kernel adds the ranges in order and writes y -- and, when qy is not
// null, quantizes it per token into codes qy [m, n] and scales y_scale [m]
// (then n <= kRequantMaxN).  tok_group_splits is the number of ranges a
// call takes (test hook FP8W8A8_TOKG_SPLITS), at most kTokGroupMaxSplits
// and at most kGroupMax - count + 1.
constexpr int kTokGroupMaxSplits = 8;
// The split item's raw sums are addressed with 32-bit offsets per range
// (m * n * 4 bytes, m <= 256): n is bounded accordingly.
constexpr int64_t kTokSplitMaxN = int64_t{1} << 20;
int tok_group_splits(const TokLinear* items, int count, int64_t m, int rq);
hipError_t launch_tok_group_requant(const TokLinear* items, int count, int64_t m, int rq,
                                    int splits, float* part, uint8_t* qy, float* y_scale,
                                    hipStream_t stream);
// Split sums part [splits, m, n] added in split order and scaled as the
// GEMM's epilogue does, y = bf16(sum * sw[n] * sx[m]) (row stride ldy);
// n % 4 == 0.
hipError_t launch_splitk_reduce(const float* part, int splits, const float* sx,
                                const float* sw, int64_t m, int64_t n, uint16_t* y,
                                int64_t ldy, hipStream_t stream);
// Split sums part [splits, m, n] added in split order, scaled as the GEMM's
// epilogue does (y = bf16(sum * sw[n] * sx[m])), written to y (row stride
// ldy) and quantized per token into q [m, n] and scale [m];
// n <= kRequantMaxN, n % 8 == 0.
hipError_t launch_splitk_reduce_quant(const float* part, int splits, const float* sx,
                                      const float* sw, int64_t m, int64_t n, uint16_t* y,
                                      int64_t ldy, uint8_t* q, float* scale,
                                      hipStream_t stream);
// The MFMA-tile permutation of a row-major [n, k] E4M3 matrix (n % 16 == 0,
// k % 128 == 0) into out (n * k bytes).
hipError_t launch_tile_weights(const uint8_t* qw, int64_t n, int64_t k, uint8_t* out,
                               hipStream_t stream);

// Token-group GEMV, kGemvMaxM < m <= kGemvTokMaxM, on quantized activations.
constexpr int kGemvTokMaxM = 64;
hipError_t launch_gemv_tok(const uint8_t* qx, const float* sx,
                           const uint8_t* qw, const float* sw, int64_t m,
                           int64_t n, int64_t k, uint16_t* y, int64_t ldy,
                           hipStream_t stream);

hipError_t launch_zero_fill(void* p, size_t bytes, hipStream_t stream);

}  // namespace fp8w8a8
