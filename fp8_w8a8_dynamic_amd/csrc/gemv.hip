// Decode-sized FP8_DYNAMIC Linear (1 <= M <= 16 tokens), bound by the HBM
// bytes of the E4M3 weights (MOSS-VL-Realtime-FP8 article, section on why
// the model is quantized: in streaming decode, memory bandwidth sets the
// response speed, and 8-bit weights halve it against BF16).
//
// Work decomposition: the output is cut into tiles of 16 output channels;
// each tile's K range is cut into `split_k` chunks; one 256-thread
// workgroup owns one (tile, chunk) and its 4 waves each stream a quarter of
// the chunk.  A wave streams its 16 weight rows straight from HBM into
// registers (32 bytes per lane per MFMA step, whole 128-byte lines per row)
// and multiplies them with v_mfma_f32_16x16x128_f8f6f4: A = 16 weight rows,
// B = the (up to 16) token rows, so the matrix cores have ample headroom
// and the kernel stays on the weight-streaming roofline.  The four waves'
// partial tiles are added in LDS in a fixed order; chunks of one tile are
// added by whichever workgroup arrives last (arrival counter), again in
// chunk order 0..split_k-1, so results are deterministic.  That workgroup
// applies the epilogue y = bf16(acc * sx[m] * sw[n]) and resets the counter
// to zero for the next call.
//
// Fused mode (bf16 activations in): every workgroup first takes the amax of
// each token row over the whole K (rows are tiny and L2-resident), derives
// the same float32 scale and quantizes its own K chunk into LDS with exactly
// the arithmetic of the stand-alone quantization kernel, while its weight
// loads are already in flight.
#include "device_common.h"
#include "launch.h"

namespace fp8w8a8 {

namespace detail {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kStepBytes = 128;        // K bytes per MFMA
constexpr int kBatch = 4;              // MFMA steps whose loads are in flight
constexpr int kLdsRowPad = 16;
constexpr int64_t kGemvFusedLds = 64 * 1024;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 16-byte streaming load of weight bytes that are read exactly once.
__device__ __forceinline__ uint4 load_stream16(const uint8_t* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ v8i to_v8i(uint4 lo, uint4 hi) {
  v8i r;
  r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
  r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
  return r;
}

template <bool FUSED>
__global__ __launch_bounds__(256) void gemv_fp8_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, const uint8_t* __restrict__ qx,
    const float* __restrict__ sx, const uint8_t* __restrict__ qw,
    const float* __restrict__ sw, int M, int N, int K, int split_k,
    int k_chunk, uint16_t* __restrict__ y, int64_t ldy,
    float* __restrict__ partials, unsigned* __restrict__ counters) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds_dyn[];
  __shared__ float red[kWaves - 1][64][4];
  __shared__ float s_scale[kGemvMaxM];
  __shared__ uint32_t s_amax[kWaves][kGemvMaxM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // Wave-uniform values live in scalar registers.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tile = blockIdx.x / split_k;
  const int chunk = blockIdx.x - tile * split_k;
  const int n0 = tile * 16;
  const int kbeg = chunk * k_chunk;
  // The chunk's 128-byte steps are dealt to the 4 waves as evenly as
  // possible (a wave may get none when the chunk is short).
  const int csteps = k_chunk / kStepBytes;
  const int s_beg = (wave * csteps) / kWaves;
  const int steps = ((wave + 1) * csteps) / kWaves - s_beg;
  const int kwoff = s_beg * kStepBytes;          // offset inside the chunk
  const int kwave = kbeg + kwoff;

  // A operand: lane -> weight row n0 + (lane & 15), 32 bytes at 32*(lane>>4)
  // of every 128-byte step.  B operand: lane -> token (lane & 15), same K
  // bytes; tokens >= M read token 0's bytes and are zeroed by a select.
  const int arow = lane & 15;
  const int kq = (lane >> 4) * 32;
  const uint8_t* wptr =
      qw + static_cast<int64_t>(n0 + arow) * K + kwave + kq;
  const int tok = lane & 15;
  const bool tok_ok = tok < M;
  const int tok_rd = tok_ok ? tok : 0;

  // Start the first batch of weight loads before anything else.
  const int nfull = steps / kBatch;              // full batches
  uint4 wa[kBatch][2];
  if (nfull > 0) {
#pragma unroll
    for (int s = 0; s < kBatch; ++s) {
      wa[s][0] = load_stream16(wptr + s * kStepBytes);
      wa[s][1] = load_stream16(wptr + s * kStepBytes + 16);
    }
  }

  const int lds_stride = k_chunk + kLdsRowPad;
  if constexpr (FUSED) {
    // 1) amax of each token row over the full K (integer max on bf16 bits).
    const int nvec = K / 8;
    for (int m = 0; m < M; ++m) {
      const uint4* xr = reinterpret_cast<const uint4*>(x + m * ldx);
      uint32_t mm = 0;
      for (int v = tid; v < nvec; v += 256) {
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
    // 2) quantize this workgroup's K chunk of every token row into LDS.
    const int cvec = k_chunk / 8;
    for (int m = 0; m < M; ++m) {
      const uint4* xr = reinterpret_cast<const uint4*>(x + m * ldx + kbeg);
      const float s = s_scale[m];
      for (int v = tid; v < cvec; v += 256)
        *reinterpret_cast<uint2*>(lds_dyn + m * lds_stride + v * 8) =
            quantize8(xr[v], s);
    }
    __syncthreads();
  }

  // B fragment of one step (k offset inside the chunk), zero for tokens >= M.
  auto load_b = [&](int koff) -> v8i {
    uint4 lo, hi;
    if constexpr (FUSED) {
      const uint8_t* p = lds_dyn + tok_rd * lds_stride + koff + kq;
      lo = *reinterpret_cast<const uint4*>(p);
      hi = *reinterpret_cast<const uint4*>(p + 16);
    } else {
      const uint8_t* p = qx + static_cast<int64_t>(tok_rd) * K + kbeg + koff + kq;
      lo = *reinterpret_cast<const uint4*>(p);
      hi = *reinterpret_cast<const uint4*>(p + 16);
    }
    v8i r = to_v8i(lo, hi);
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = tok_ok ? r[i] : 0;
    return r;
  };

  v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int b = 0; b < nfull; ++b) {
    v8i wfrag[kBatch];
#pragma unroll
    for (int s = 0; s < kBatch; ++s) wfrag[s] = to_v8i(wa[s][0], wa[s][1]);
    if (b + 1 < nfull) {
      const uint8_t* nxt = wptr + (b + 1) * kBatch * kStepBytes;
#pragma unroll
      for (int s = 0; s < kBatch; ++s) {
        wa[s][0] = load_stream16(nxt + s * kStepBytes);
        wa[s][1] = load_stream16(nxt + s * kStepBytes + 16);
      }
    }
#pragma unroll
    for (int s = 0; s < kBatch; ++s) {
      const v8i xb = load_b(kwoff + (b * kBatch + s) * kStepBytes);
      acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
          wfrag[s], xb, acc, 0, 0, 0, 0, 0, 0);
    }
  }
  for (int s = nfull * kBatch; s < steps; ++s) {
    const v8i wf = to_v8i(load_stream16(wptr + s * kStepBytes),
                          load_stream16(wptr + s * kStepBytes + 16));
    const v8i xb = load_b(kwoff + s * kStepBytes);
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf, xb, acc, 0, 0,
                                                           0, 0, 0, 0);
  }

  // Add the 4 waves' tiles in wave order.  16x16 accumulator layout: lane
  // holds column (lane & 15) = token and rows 4*(lane>>4) + r = channel.
  if (wave > 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave - 1][lane][r] = acc[r];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < kWaves - 1; ++w)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] += red[w][lane][r];

  if (split_k > 1) {
    // Hand-off between the workgroups of one tile without whole-cache
    // flushes: partials are written and read with device-coherent (sc1)
    // accesses, which bypass the per-XCD caches; the writer waits for its
    // stores to complete before bumping the arrival counter, and only the
    // last arriver, which has seen every other increment, reads them.
    float* mine = partials + (static_cast<int64_t>(tile) * split_k + chunk) * 256;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      __hip_atomic_store(mine + lane * 4 + r, acc[r], __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0x0F70);          // vmcnt(0): stores done
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    unsigned prev = 0;
    if (lane == 0)
      prev = __hip_atomic_fetch_add(counters + tile, 1u, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT);
    prev = __shfl(prev, 0, 64);
    if (prev != static_cast<unsigned>(split_k - 1)) return;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    v4f sum = {0.0f, 0.0f, 0.0f, 0.0f};
    const float* all = partials + static_cast<int64_t>(tile) * split_k * 256;
    for (int c = 0; c < split_k; ++c) {
      if (c == chunk) {
        sum += acc;
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          sum[r] += __hip_atomic_load(all + c * 256 + lane * 4 + r,
                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    acc = sum;
    if (lane == 0)
      __hip_atomic_store(counters + tile, 0u, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }

  if (!tok_ok) return;
  const float xs = FUSED ? s_scale[tok] : sx[tok];
  const int nb0 = n0 + 4 * (lane >> 4);
  const float4 ws = *reinterpret_cast<const float4*>(sw + nb0);
  uint2 out;
  out.x = pack_bf16x2(acc[0] * xs * ws.x, acc[1] * xs * ws.y);
  out.y = pack_bf16x2(acc[2] * xs * ws.z, acc[3] * xs * ws.w);
  *reinterpret_cast<uint2*>(y + static_cast<int64_t>(tok) * ldy + nb0) = out;
}

}  // namespace detail
using namespace detail;

GemvPlan plan_gemv(int64_t m, int64_t n, int64_t k, bool fused) {
  const int64_t tiles = n / 16;
  int split = 1;
  // Halve the K chunk while it stays a whole number of 128-byte steps and at
  // least one step per wave, until there are >= 512 workgroups (two per CU).
  auto can_halve = [&](int s) {
    return k % (static_cast<int64_t>(kStepBytes) * s * 2) == 0 &&
           k / (s * 2) >= kWaves * kStepBytes;
  };
  while (tiles * split < 512 && tiles <= kMaxSplitTiles && can_halve(split))
    split *= 2;
  // Fused mode keeps M x chunk bytes of codes in LDS: at most 64 KiB.
  while (fused && m * (k / split + kLdsRowPad) > kGemvFusedLds &&
         tiles <= kMaxSplitTiles &&
         k % (static_cast<int64_t>(kStepBytes) * split * 2) == 0)
    split *= 2;
  return GemvPlan{split, static_cast<int>(k / split)};
}

bool gemv_fused_fits(int64_t m, int64_t n, int64_t k) {
  const GemvPlan p = plan_gemv(m, n, k, true);
  return m * (p.k_chunk + kLdsRowPad) <= kGemvFusedLds;
}

size_t gemv_partial_bytes(int64_t m, int64_t n, int64_t k, bool fused) {
  const GemvPlan p = plan_gemv(m, n, k, fused);
  if (p.split_k <= 1) return 0;
  return static_cast<size_t>(n / 16) * p.split_k * 256 * 4;
}

hipError_t launch_gemv(const uint16_t* x, int64_t ldx, const uint8_t* qx,
                       const float* sx, const uint8_t* qw, const float* sw,
                       int64_t m, int64_t n, int64_t k, uint16_t* y,
                       int64_t ldy, unsigned* counters, float* partials,
                       hipStream_t stream) {
  if (m == 0 || n == 0) return hipSuccess;
  const bool fused = x != nullptr;
  const GemvPlan p = plan_gemv(m, n, k, fused);
  const int64_t tiles = n / 16;
  const dim3 grid(static_cast<uint32_t>(tiles * p.split_k));
  if (fused) {
    const size_t lds = static_cast<size_t>(m) * (p.k_chunk + kLdsRowPad);
    gemv_fp8_kernel<true><<<grid, dim3(256), lds, stream>>>(
        x, ldx, qx, sx, qw, sw, static_cast<int>(m), static_cast<int>(n), static_cast<int>(k), p.split_k, p.k_chunk, y, ldy, partials, counters);
  } else {
    gemv_fp8_kernel<false><<<grid, dim3(256), 0, stream>>>(
        x, ldx, qx, sx, qw, sw, static_cast<int>(m), static_cast<int>(n), static_cast<int>(k), p.split_k, p.k_chunk, y, ldy, partials, counters);
  }
  return hipGetLastError();
}

}  // namespace fp8w8a8
