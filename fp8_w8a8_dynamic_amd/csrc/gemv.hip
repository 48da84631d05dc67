// Decode-sized FP8_DYNAMIC Linear (1 <= M <= 16 tokens), bound by the HBM
// bytes of the E4M3 weights (MOSS-VL-Realtime-FP8 article, section on why
// the model is quantized: in streaming decode, memory bandwidth sets the
// response speed, and 8-bit weights halve it against BF16).
//
// Work decomposition: one workgroup of kWaves waves owns a tile of 16 output
// channels and streams those 16 weight rows over the whole K; the K range is
// dealt to its waves in 128-byte steps.  A wave issues the loads of all its
// steps (up to kMaxSteps) at once, straight from HBM into registers: 32
// bytes per lane per step, so each step reads whole 128-byte lines of the 16
// rows.  Each step is one v_mfma_f32_16x16x128_f8f6f4 with A = the 16 weight
// rows and B = the (up to 16) token rows of the activation codes; the matrix
// cores have far more throughput than the weight stream needs.  The waves'
// 16x16 partial tiles are added in LDS in wave order (deterministic), and
// wave 0 applies the epilogue y = bf16(acc * sx[m] * sw[n]).  No workgroup
// ever waits on another: there is no cross-workgroup reduction.
//
// Fused mode (bf16 activations in, M small): while its weight loads are in
// flight the workgroup takes the amax of each token row over the whole K
// (integer max on bf16 bits), derives the float32 scale and quantizes the
// rows into LDS with exactly the arithmetic of the stand-alone quantization
// kernel; the B operands are then read from LDS.
#include <cstdlib>

#include "device_common.h"
#include "launch.h"

namespace fp8w8a8 {

namespace detail {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kStepBytes = 128;        // K bytes per MFMA
constexpr int kLdsRowPad = 16;
constexpr int64_t kGemvFusedLds = 64 * 1024;

// 16-byte load of weight bytes.  (Plain loads: the two loads of a step
// touch the same 128-byte lines, and a non-temporal hint could let the line
// leave L2 between them.)
__device__ __forceinline__ uint4 load16(const uint8_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

__device__ __forceinline__ v8i to_v8i(uint4 lo, uint4 hi) {
  v8i r;
  r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
  r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
  return r;
}

// WAVES waves per workgroup; each wave keeps the loads of up to MAXSTEPS
// 128-byte steps in flight.
template <bool FUSED, int WAVES, int MAXSTEPS>
__global__ __launch_bounds__(WAVES * 64) void gemv_fp8_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, const uint8_t* __restrict__ qx,
    const float* __restrict__ sx, const uint8_t* __restrict__ qw,
    const float* __restrict__ sw, int M, int K, uint16_t* __restrict__ y,
    int64_t ldy) {
  constexpr int kWaves = WAVES;
  constexpr int kThreads = WAVES * 64;
  constexpr int kMaxSteps = MAXSTEPS;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds_x[];
  __shared__ float red[kWaves][64][4];
  __shared__ float s_scale[kGemvMaxM];
  __shared__ uint32_t s_amax[kWaves][kGemvMaxM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n0 = blockIdx.x * 16;
  // The K range's 128-byte steps, dealt to the waves as evenly as possible.
  const int csteps = K / kStepBytes;
  const int s_beg = (wave * csteps) / kWaves;
  const int steps = ((wave + 1) * csteps) / kWaves - s_beg;

  // A operand: lane -> weight row n0 + (lane & 15); its 32 bytes of every
  // 128-byte step are bytes [16g, 16g+16) and [64+16g, 64+16g+16) with
  // g = lane >> 4, so each of the two 16-byte loads of a step reads 64
  // contiguous bytes of every row.  (Which K index sits in which operand byte
  // is free as long as A and B agree.)  B operand: lane -> token (lane & 15),
  // same K bytes; tokens >= M read token 0's bytes and are zeroed.
  const int kq = (lane >> 4) * 16;
  const uint8_t* wptr = qw + static_cast<int64_t>(n0 + (lane & 15)) * K +
                        s_beg * kStepBytes + kq;
  const int tok = lane & 15;
  const bool tok_ok = tok < M;
  const int tok_rd = tok_ok ? tok : 0;

  // Issue the first batch of weight loads before anything else.
  uint4 wa[kMaxSteps][2];
#pragma unroll
  for (int s = 0; s < kMaxSteps; ++s)
    if (s < steps) {
      wa[s][0] = load16(wptr + s * kStepBytes);
      wa[s][1] = load16(wptr + s * kStepBytes + 64);
    }

  const int lds_stride = K + kLdsRowPad;
  if constexpr (FUSED) {
    // 1) amax of each token row over the full K (integer max on bf16 bits).
    const int nvec = K / 8;
    for (int m = 0; m < M; ++m) {
      const uint4* xr = reinterpret_cast<const uint4*>(x + m * ldx);
      uint32_t mm = 0;
      for (int v = tid; v < nvec; v += kThreads) {
        const uint4 t = xr[v];
        mm = pk_max_u16(mm, bf16x2_abs_bits(t.x));
        mm = pk_max_u16(mm, bf16x2_abs_bits(t.y));
        mm = pk_max_u16(mm, bf16x2_abs_bits(t.z));
        mm = pk_max_u16(mm, bf16x2_abs_bits(t.w));
      }
      const uint32_t wmax = wave_max_u32(max(mm & 0xffffu, mm >> 16));
      if (lane == 0) s_amax[wave][m] = wmax;
    }
    __syncthreads();
    if (tid < M) {
      uint32_t a = s_amax[0][tid];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) a = max(a, s_amax[w][tid]);
      s_scale[tid] = row_scale(__uint_as_float(a << 16));
    }
    __syncthreads();
    // 2) quantize every token row into LDS (codes, row stride K + pad).
    for (int m = 0; m < M; ++m) {
      const uint4* xr = reinterpret_cast<const uint4*>(x + m * ldx);
      const float s = s_scale[m];
      for (int v = tid; v < nvec; v += kThreads)
        *reinterpret_cast<uint2*>(lds_x + m * lds_stride + v * 8) =
            quantize8(xr[v], s);
    }
    __syncthreads();
  }

  // B fragment of one step (k offset within the row), zero for tokens >= M.
  auto load_b = [&](int koff) -> v8i {
    uint4 lo, hi;
    if constexpr (FUSED) {
      const uint8_t* p = lds_x + tok_rd * lds_stride + koff + kq;
      lo = *reinterpret_cast<const uint4*>(p);
      hi = *reinterpret_cast<const uint4*>(p + 64);
    } else {
      const uint8_t* p = qx + static_cast<int64_t>(tok_rd) * K + koff + kq;
      lo = *reinterpret_cast<const uint4*>(p);
      hi = *reinterpret_cast<const uint4*>(p + 64);
    }
    v8i r = to_v8i(lo, hi);
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = tok_ok ? r[i] : 0;
    return r;
  };

  v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int base = 0; base < steps; base += kMaxSteps) {
    v8i wf[kMaxSteps];
#pragma unroll
    for (int s = 0; s < kMaxSteps; ++s) wf[s] = to_v8i(wa[s][0], wa[s][1]);
    // Next batch's loads go out before this batch's MFMAs.
    const int nb = base + kMaxSteps;
#pragma unroll
    for (int s = 0; s < kMaxSteps; ++s)
      if (nb + s < steps) {
        wa[s][0] = load16(wptr + (nb + s) * kStepBytes);
        wa[s][1] = load16(wptr + (nb + s) * kStepBytes + 64);
      }
#pragma unroll
    for (int s = 0; s < kMaxSteps; ++s)
      if (base + s < steps) {
        const v8i xb = load_b((s_beg + base + s) * kStepBytes);
        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            wf[s], xb, acc, 0, 0, 0, 0, 0, 0);
      }
  }

  // Add the waves' tiles in wave order.  16x16 accumulator layout: lane
  // holds column (lane & 15) = token and rows 4*(lane>>4) + r = channel.
#pragma unroll
  for (int r = 0; r < 4; ++r) red[wave][lane][r] = acc[r];
  __syncthreads();
  if (wave != 0) return;
  v4f sum = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int w = 0; w < kWaves; ++w)
#pragma unroll
    for (int r = 0; r < 4; ++r) sum[r] += red[w][lane][r];
  if (!tok_ok) return;
  const float xs = FUSED ? s_scale[tok] : sx[tok];
  const int nb0 = n0 + 4 * (lane >> 4);
  const float4 ws = *reinterpret_cast<const float4*>(sw + nb0);
  uint2 out;
  out.x = pack_bf16x2(sum[0] * ws.x * xs, sum[1] * ws.y * xs);
  out.y = pack_bf16x2(sum[2] * ws.z * xs, sum[3] * ws.w * xs);
  *reinterpret_cast<uint2*>(y + static_cast<int64_t>(tok) * ldy + nb0) = out;
}

}  // namespace detail
using namespace detail;

bool gemv_fused_fits(int64_t m, int64_t n, int64_t k) {
  (void)n;
  return m * (k + kLdsRowPad) <= kGemvFusedLds;
}

template <bool FUSED, int WAVES, int MAXSTEPS>
hipError_t launch_one(const uint16_t* x, int64_t ldx, const uint8_t* qx,
                      const float* sx, const uint8_t* qw, const float* sw,
                      int64_t m, int64_t n, int64_t k, uint16_t* y,
                      int64_t ldy, hipStream_t stream) {
  const dim3 grid(static_cast<uint32_t>(n / 16));
  const size_t lds = FUSED ? static_cast<size_t>(m) * (k + kLdsRowPad) : 0;
  gemv_fp8_kernel<FUSED, WAVES, MAXSTEPS><<<grid, dim3(WAVES * 64), lds, stream>>>(
      x, ldx, qx, sx, qw, sw, static_cast<int>(m), static_cast<int>(k), y, ldy);
  return hipGetLastError();
}

hipError_t launch_gemv(const uint16_t* x, int64_t ldx, const uint8_t* qx,
                       const float* sx, const uint8_t* qw, const float* sw,
                       int64_t m, int64_t n, int64_t k, uint16_t* y,
                       int64_t ldy, hipStream_t stream) {
  if (m == 0 || n == 0) return hipSuccess;
  // Many tiles: small workgroups, several resident per CU, each wave with a
  // deep queue of loads.  Few tiles: one wide workgroup per tile so that the
  // tile's K range is streamed by 16 waves at once.
  int variant = n / 16 >= 512 ? 0 : 1;
  if (const char* e = std::getenv("FP8W8A8_GEMV_VARIANT")) variant = std::atoi(e) & 1;
  const bool fused = x != nullptr;
  if (variant == 0)
    return fused ? launch_one<true, 4, 8>(x, ldx, qx, sx, qw, sw, m, n, k, y, ldy, stream)
                 : launch_one<false, 4, 8>(x, ldx, qx, sx, qw, sw, m, n, k, y, ldy, stream);
  return fused ? launch_one<true, 16, 4>(x, ldx, qx, sx, qw, sw, m, n, k, y, ldy, stream)
               : launch_one<false, 16, 4>(x, ldx, qx, sx, qw, sw, m, n, k, y, ldy, stream);
}

}  // namespace fp8w8a8
