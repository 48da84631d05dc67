// Prefill FP8 x FP8 GEMM with the token-scale x channel-scale epilogue
// (MOSS-VL quantization README, "FP8-Dynamic" recipe: FP8 per-token
// activations times float8_e4m3fn channel-wise weights in "the quantized
// kernels", output back to bfloat16).
//
//   y[m,n] = bf16_rne( (sum_k dec(qx[m,k]) * dec(qw[n,k])) * sx[m] * sw[n] )
//
// Both operands are K-contiguous ("NT"), which is what the MFMA operand
// fragments want.  Design for gfx950:
//   * v_mfma_f32_32x32x64_f8f6f4 (E4M3 x E4M3 -> f32; every product is exact
//     in f32, accumulation in f32);
//   * a 256-thread workgroup (4 waves in 2x2) owns a BM x BN output tile;
//     each wave owns (BM/2) x (BN/2) and keeps it in registers;
//   * K advances 128 bytes per stage; stages are double-buffered in LDS and
//     filled with global_load_lds_dwordx4 (HBM/L2 -> LDS without passing
//     through VGPRs) while the MFMAs consume the other stage;
//   * LDS rows are 128 bytes with the 16-byte chunk index XOR-swizzled by
//     (row & 7), so the ds_read_b128 of 8 consecutive rows hit 8 different
//     bank groups; the swizzle is applied on the global side (each lane
//     fetches the chunk that belongs at its fixed LDS slot);
//   * workgroup -> tile mapping is XCD-aware: the hardware deals workgroups
//     round-robin over the 8 XCDs, so consecutive logical tiles (which share
//     operand rows in groups of 4 tile-rows) are given to one XCD and its L2.
// Rows beyond M or N are loaded clamped to the last valid row and never
// stored.  K must be a multiple of 128.
#include "device_common.h"
#include "launch.h"

namespace fp8w8a8 {

namespace detail {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kBK = 128;  // bytes of K per stage
constexpr int kGroupM = 4;

template <int BM, int BN>
struct GemmShape {
  static constexpr int WM = BM / 2, WN = BN / 2;    // wave tile
  static constexpr int TM = WM / 32, TN = WN / 32;  // 32x32 MFMA tiles
  static constexpr int A_STAGE = BM * kBK, B_STAGE = BN * kBK;
  static constexpr int STAGE = A_STAGE + B_STAGE;
  static constexpr int LDS = 2 * STAGE;
  static constexpr int A_LOADS = BM / 32;  // 1 KB loads per wave per stage
  static constexpr int B_LOADS = BN / 32;
};

__device__ __forceinline__ void map_tile(int bid, int tiles_m, int tiles_n,
                                         int& tm, int& tn) {
  const int total = tiles_m * tiles_n;
  int lid = bid;
  const int per_xcd = total / 8;
  if (bid < per_xcd * 8) lid = (bid % 8) * per_xcd + bid / 8;
  const int per_group = kGroupM * tiles_n;
  const int g = lid / per_group;
  const int first_m = g * kGroupM;
  const int gsize = min(tiles_m - first_m, kGroupM);
  const int in = lid - g * per_group;
  tm = first_m + in % gsize;
  tn = in / gsize;
}

__device__ __forceinline__ v8i lds_frag(const uint8_t* base, int p0) {
  const uint4 lo = *reinterpret_cast<const uint4*>(base + p0 * 16);
  const uint4 hi = *reinterpret_cast<const uint4*>(base + (p0 ^ 1) * 16);
  v8i r;
  r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
  r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
  return r;
}

typedef int v4i __attribute__((ext_vector_type(4)));

// Buffer resource for `bytes` bytes at `base` (raw buffer, stride 0).  Loads
// at offsets >= bytes return zero: this is how rows past M or N read as 0.
__device__ __forceinline__ v4i make_rsrc(const uint8_t* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  v4i r;
  r[0] = static_cast<int>(static_cast<uint32_t>(a));
  r[1] = static_cast<int>(static_cast<uint32_t>(a >> 32) & 0xffffu);
  r[2] = static_cast<int>(bytes);
  r[3] = 0x00020000;  // raw 32-bit data format, no swizzle
  return r;
}

// One 16-byte-per-lane copy global -> LDS (buffer_load_dwordx4 ... lds): the
// wave's 64 x 16 bytes land contiguously at LDS byte address `lds` (M0).
// Inline asm because the compiler's wait-count insertion cannot tell the two
// stage buffers apart and would serialize every copy with the MFMAs on the
// other stage.  The instruction has no register result; the kernel waits for
// the copies explicitly (vmcnt(0) + barrier) before reading the stage.
__device__ __forceinline__ void lds_copy16(v4i rsrc, uint32_t voff,
                                           uint32_t soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(soff), "s"(lds)
               : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)p));
}

template <int BM, int BN, int MINB>
__global__ __launch_bounds__(256, MINB) void gemm_fp8_kernel(
    const uint8_t* __restrict__ qx, const float* __restrict__ sx,
    const uint8_t* __restrict__ qw, const float* __restrict__ sw, int M,
    int N, int K, uint16_t* __restrict__ y, int64_t ldy, int tiles_m,
    int tiles_n) {
  using S = GemmShape<BM, BN>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[S::LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  int tm, tn;
  map_tile(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  // Descriptors cover exactly this tile's valid rows.
  const v4i a_rsrc = make_rsrc(qx + static_cast<int64_t>(m0) * K,
                               static_cast<uint32_t>(min(M - m0, BM)) * K);
  const v4i b_rsrc = make_rsrc(qw + static_cast<int64_t>(n0) * K,
                               static_cast<uint32_t>(min(N - n0, BN)) * K);

  // Global -> LDS assignment.  One wave instruction fills 1 KB of LDS =
  // 8 rows x 128 bytes; lane j lands at byte 16*j: row j>>3, physical chunk
  // j&7, which holds logical chunk (j&7) ^ (row&7).
  const int lrow = lane >> 3;
  const int lchunk = (lane & 7) ^ lrow;
  uint32_t a_off[S::A_LOADS], b_off[S::B_LOADS];
#pragma unroll
  for (int i = 0; i < S::A_LOADS; ++i)
    a_off[i] = static_cast<uint32_t>(((wave * S::A_LOADS + i) * 8 + lrow) * K +
                                     lchunk * 16);
#pragma unroll
  for (int i = 0; i < S::B_LOADS; ++i)
    b_off[i] = static_cast<uint32_t>(((wave * S::B_LOADS + i) * 8 + lrow) * K +
                                     lchunk * 16);
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(smem));
  const uint32_t a_lds = lds0 + wave * S::A_LOADS * 1024;
  const uint32_t b_lds = lds0 + S::A_STAGE + wave * S::B_LOADS * 1024;

  v16f acc[S::TM][S::TN];
#pragma unroll
  for (int t = 0; t < S::TM; ++t)
#pragma unroll
    for (int u = 0; u < S::TN; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[t][u][r] = 0.0f;

  // Fragment addressing: lane reads row (lane & 31) of each 32-row tile and
  // K half (lane >> 5) of each 64-byte MFMA step: logical chunks c, c+1 with
  // c = 4*step + 2*(lane>>5); physical chunk = logical ^ (row & 7).
  const int frow = lane & 31;
  const int fhalf = lane >> 5;
  const int a_row0 = wm * S::WM + frow;
  const int b_row0 = wn * S::WN + frow;

  const int KT = K / kBK;
  auto issue = [&](int st, int k0) {
    const uint32_t so = static_cast<uint32_t>(k0);
#pragma unroll
    for (int i = 0; i < S::A_LOADS; ++i)
      lds_copy16(a_rsrc, a_off[i], so, a_lds + st * S::STAGE + i * 1024);
#pragma unroll
    for (int i = 0; i < S::B_LOADS; ++i)
      lds_copy16(b_rsrc, b_off[i], so, b_lds + st * S::STAGE + i * 1024);
  };
  issue(0, 0);
  for (int kt = 0; kt < KT; ++kt) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's copies landed
    __syncthreads();                     // all copies landed; the other stage
                                         // is no longer being read
    if (kt + 1 < KT) issue((kt + 1) & 1, (kt + 1) * kBK);
    const uint8_t* as = smem + (kt & 1) * S::STAGE;
    const uint8_t* bs = as + S::A_STAGE;
#pragma unroll
    for (int step = 0; step < 2; ++step) {
      const int p0 = (4 * step + 2 * fhalf) ^ (frow & 7);
      v8i af[S::TM], bf[S::TN];
#pragma unroll
      for (int t = 0; t < S::TM; ++t)
        af[t] = lds_frag(as + (a_row0 + 32 * t) * kBK, p0);
#pragma unroll
      for (int u = 0; u < S::TN; ++u)
        bf[u] = lds_frag(bs + (b_row0 + 32 * u) * kBK, p0);
#pragma unroll
      for (int t = 0; t < S::TM; ++t)
#pragma unroll
        for (int u = 0; u < S::TN; ++u)
          acc[t][u] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              af[t], bf[u], acc[t][u], 0, 0, 0, 0, 0, 0);
    }
  }

  // Epilogue.  32x32 accumulator layout: lane holds column (lane & 31) and
  // rows 8*(r>>2) + 4*(lane>>5) + (r&3), r = 0..15.
#pragma unroll
  for (int t = 0; t < S::TM; ++t) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int gm = m0 + wm * S::WM + 32 * t + 8 * (r >> 2) + 4 * fhalf + (r & 3);
      if (gm >= M) continue;
      const float xs = sx[gm];
      uint16_t* yrow = y + static_cast<int64_t>(gm) * ldy;
#pragma unroll
      for (int u = 0; u < S::TN; ++u) {
        const int gn = n0 + wn * S::WN + 32 * u + frow;
        if (gn < N) yrow[gn] = f32_to_bf16_bits(acc[t][u][r] * xs * sw[gn]);
      }
    }
  }
}

template <int BM, int BN, int MINB>
hipError_t launch_cfg(const uint8_t* qx, const float* sx, const uint8_t* qw,
                      const float* sw, int64_t m, int64_t n, int64_t k,
                      uint16_t* y, int64_t ldy, hipStream_t stream) {
  const int tiles_m = static_cast<int>((m + BM - 1) / BM);
  const int tiles_n = static_cast<int>((n + BN - 1) / BN);
  gemm_fp8_kernel<BM, BN, MINB><<<dim3(static_cast<uint32_t>(tiles_m * tiles_n)), dim3(256), 0, stream>>>(
        qx, sx, qw, sw, static_cast<int>(m), static_cast<int>(n), static_cast<int>(k), y, ldy, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace detail
using namespace detail;

hipError_t launch_gemm(const uint8_t* qx, const float* sx, const uint8_t* qw,
                       const float* sw, int64_t m, int64_t n, int64_t k,
                       uint16_t* y, int64_t ldy, hipStream_t stream) {
  if (m == 0 || n == 0) return hipSuccess;
  const int64_t big_tiles = ((m + 255) / 256) * ((n + 255) / 256);
  if (big_tiles >= 192)
    return launch_cfg<256, 256, 1>(qx, sx, qw, sw, m, n, k, y, ldy, stream);
  return launch_cfg<128, 128, 2>(qx, sx, qw, sw, m, n, k, y, ldy, stream);
}

}  // namespace fp8w8a8
