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
#include <cstdlib>

#include "device_common.h"
#include "launch.h"

namespace fp8w8a8 {

namespace detail {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kGroupM = 4;

// Tile configuration: BM x BN output tile per 256-thread workgroup (4 waves
// in 2x2, each owning (BM/2) x (BN/2)), BK bytes of K per LDS stage, STAGES
// stage buffers (copies run STAGES-1 stages ahead of the MFMAs).
template <int BM, int BN, int BK, int STAGES>
struct GemmShape {
  static constexpr int WM = BM / 2, WN = BN / 2;    // wave tile
  static constexpr int TM = WM / 32, TN = WN / 32;  // 32x32 MFMA tiles
  static constexpr int CH = BK / 16;                // 16-byte chunks per row
  static constexpr int RPI = 1024 / BK;             // rows per 1 KB copy
  static constexpr int A_STAGE = BM * BK, B_STAGE = BN * BK;
  static constexpr int STAGE = A_STAGE + B_STAGE;
  static constexpr int LDS = STAGES * STAGE;
  static constexpr int A_LOADS = A_STAGE / 4096;    // 1 KB copies per wave
  static constexpr int B_LOADS = B_STAGE / 4096;
  static constexpr int STEPS = BK / 64;             // MFMA K-steps per stage
  // Epilogue staging: each wave's WM x WN bf16 tile, rows padded by 16 B.
  static constexpr int EPI_ROW = WN * 2 + 16;
  static constexpr int EPI = 4 * WM * EPI_ROW;
  static constexpr int SMEM = LDS > EPI ? LDS : EPI;
  static_assert(BK == 64 || BK == 128, "BK is 64 or 128 bytes");
  static_assert(STAGES >= 2 && STAGES <= 4, "2..4 stages");
  static_assert(SMEM <= 160 * 1024, "LDS budget of one CU");
};

// XOR swizzle of the 16-byte chunk index within a row.  gfx950's LDS serves
// a ds_read_b128 16 lanes at a time from 64 four-byte banks (256 bytes), and
// the 16 lanes of a fragment read read 16 consecutive rows at the same
// logical chunk: the swizzle makes their 16 addresses fall in 16 distinct
// 16-byte bank groups.  128-byte rows: 2 rows per 256 bytes, 8 chunk values;
// 64-byte rows: 4 rows per 256 bytes, 4 chunk values.
template <int BK>
__device__ __forceinline__ int swz(int row) {
  if constexpr (BK == 128) return (row >> 1) & 7;
  else return (row >> 2) & 3;
}

// s_waitcnt immediate for "at most n vector-memory operations outstanding"
// (gfx9 encoding; expcnt and lgkmcnt left at their maxima).
constexpr int vmcnt_imm(int n) {
  return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8);
}

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

template <int BM, int BN, int BK, int STAGES, int MINB>
__global__ __launch_bounds__(256, MINB) void gemm_fp8_kernel(
    const uint8_t* __restrict__ qx, const float* __restrict__ sx,
    const uint8_t* __restrict__ qw, const float* __restrict__ sw, int M,
    int N, int K, uint16_t* __restrict__ y, int64_t ldy, int tiles_m,
    int tiles_n) {
  using S = GemmShape<BM, BN, BK, STAGES>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[S::SMEM];

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

  // Global -> LDS assignment.  One wave copy fills 1 KB of LDS = RPI rows of
  // BK bytes; lane j lands at byte 16*j: row j / CH, physical chunk j % CH,
  // which holds logical chunk (j % CH) ^ swz(row).
  uint32_t a_off[S::A_LOADS], b_off[S::B_LOADS];
#pragma unroll
  for (int i = 0; i < S::A_LOADS; ++i) {
    const int r = (wave * S::A_LOADS + i) * S::RPI + lane / S::CH;
    a_off[i] = static_cast<uint32_t>(
        r * K + (((lane % S::CH) ^ swz<BK>(r)) * 16));
  }
#pragma unroll
  for (int i = 0; i < S::B_LOADS; ++i) {
    const int r = (wave * S::B_LOADS + i) * S::RPI + lane / S::CH;
    b_off[i] = static_cast<uint32_t>(
        r * K + (((lane % S::CH) ^ swz<BK>(r)) * 16));
  }
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
  // c = 4*step + 2*(lane>>5); physical chunk = logical ^ swz(row), and
  // swz(row) depends only on (lane & 31) because tile rows start at
  // multiples of 32.
  const int frow = lane & 31;
  const int fhalf = lane >> 5;
  const int fswz = swz<BK>(frow);
  const int a_row0 = wm * S::WM + frow;
  const int b_row0 = wn * S::WN + frow;

  const int KT = K / BK;
  constexpr int PER_STAGE = S::A_LOADS + S::B_LOADS;  // copies per wave
  auto issue = [&](int st, int k0) {
    const uint32_t so = static_cast<uint32_t>(k0);
#pragma unroll
    for (int i = 0; i < S::A_LOADS; ++i)
      lds_copy16(a_rsrc, a_off[i], so, a_lds + st * S::STAGE + i * 1024);
#pragma unroll
    for (int i = 0; i < S::B_LOADS; ++i)
      lds_copy16(b_rsrc, b_off[i], so, b_lds + st * S::STAGE + i * 1024);
  };
  // Prologue: the first STAGES-1 stages.
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < KT) issue(s, s * BK);
  for (int kt = 0; kt < KT; ++kt) {
    // Wait until this wave's copies of stage kt have landed: the copies of
    // the (up to STAGES-2) later stages may stay in flight.
    const int later = min(STAGES - 2, KT - 1 - kt);
    if (later >= 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * PER_STAGE));
    else if (later == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(PER_STAGE));
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();  // all waves' copies of stage kt landed, and every wave
                      // is done reading the stage the next copy overwrites
    const uint8_t* as = smem + (kt % STAGES) * S::STAGE;
    const uint8_t* bs = as + S::A_STAGE;
    // All fragments of the stage are read first; the next stage's copies are
    // issued while those reads are in flight; then the MFMAs run back to back
    // with no LDS latency between them.
    v8i af[S::STEPS][S::TM], bf[S::STEPS][S::TN];
#pragma unroll
    for (int t = 0; t < S::TM; ++t)
      af[0][t] = lds_frag(as + (a_row0 + 32 * t) * BK, (2 * fhalf) ^ fswz);
#pragma unroll
    for (int u = 0; u < S::TN; ++u)
      bf[0][u] = lds_frag(bs + (b_row0 + 32 * u) * BK, (2 * fhalf) ^ fswz);
    if (kt + STAGES - 1 < KT)
      issue((kt + STAGES - 1) % STAGES, (kt + STAGES - 1) * BK);
    // Step 0's MFMAs alternate with the LDS reads of step 1 (when the stage
    // has two steps), so those reads are in flight under the MFMAs.
    if constexpr (S::STEPS == 2) {
      const int p1 = (4 + 2 * fhalf) ^ fswz;
#pragma unroll
      for (int t = 0; t < S::TM; ++t)
        af[1][t] = lds_frag(as + (a_row0 + 32 * t) * BK, p1);
#pragma unroll
      for (int u = 0; u < S::TN; ++u)
        bf[1][u] = lds_frag(bs + (b_row0 + 32 * u) * BK, p1);
    }
#pragma unroll
    for (int t = 0; t < S::TM; ++t)
#pragma unroll
      for (int u = 0; u < S::TN; ++u)
        acc[t][u] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            bf[0][u], af[0][t], acc[t][u], 0, 0, 0, 0, 0, 0);
    if constexpr (S::STEPS == 2) {
      constexpr int kReads = 2 * (S::TM + S::TN);      // ds_read_b128 count
      constexpr int kMfma = S::TM * S::TN;
#pragma unroll
      for (int i = 0; i < kMfma; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
        if (i < kReads) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one DS read
      }
      if (kReads > kMfma) __builtin_amdgcn_sched_group_barrier(0x100, kReads - kMfma, 0);
#pragma unroll
      for (int t = 0; t < S::TM; ++t)
#pragma unroll
        for (int u = 0; u < S::TN; ++u)
          acc[t][u] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              bf[1][u], af[1][t], acc[t][u], 0, 0, 0, 0, 0, 0);
    }
  }

  // Epilogue.  The MFMAs ran with the weight fragment as the A operand, so
  // in the 32x32 accumulator layout a lane holds one token, (lane & 31) of
  // its token tile t, and for each group q = r >> 2 four consecutive output
  // channels 8q + 4*(lane >> 5) + (r & 3) of channel tile u.  Each lane
  // scales its values, packs four bf16 (8 bytes) into this wave's region of
  // LDS laid out [token][channel], and the wave then writes whole rows back
  // with 16-byte stores (coalesced row segments of 2*WN bytes).
  __syncthreads();  // every wave is done with the stage buffers
  uint8_t* ep = smem + wave * (S::WM * S::EPI_ROW);
  const int tok0 = m0 + wm * S::WM;
  const int ch0 = n0 + wn * S::WN;
  // Channel scales of this lane: 4 consecutive channels per (u, q).
  float4 ws[S::TN][4];
#pragma unroll
  for (int u = 0; u < S::TN; ++u)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = ch0 + 32 * u + 8 * q + 4 * fhalf;
      ws[u][q] = c < N ? *reinterpret_cast<const float4*>(sw + c)
                       : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
  for (int t = 0; t < S::TM; ++t) {
    const int tl = 32 * t + frow;                    // token inside the wave tile
    const float xs = tok0 + tl < M ? sx[tok0 + tl] : 0.0f;
#pragma unroll
    for (int u = 0; u < S::TN; ++u) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int cl = 32 * u + 8 * q + 4 * fhalf;   // channel inside the tile
        uint2 pk;
        pk.x = pack_bf16x2(acc[t][u][4 * q + 0] * ws[u][q].x * xs,
                           acc[t][u][4 * q + 1] * ws[u][q].y * xs);
        pk.y = pack_bf16x2(acc[t][u][4 * q + 2] * ws[u][q].z * xs,
                           acc[t][u][4 * q + 3] * ws[u][q].w * xs);
        *reinterpret_cast<uint2*>(ep + tl * S::EPI_ROW + cl * 2) = pk;
      }
    }
  }
  // Read back whole rows: CPR 16-byte chunks per row, RPW rows per pass.
  constexpr int CPR = S::WN * 2 / 16;
  constexpr int RPW = 64 / CPR;
  const int rr = lane / CPR, cc = lane % CPR;
#pragma unroll 4
  for (int row = rr; row < S::WM; row += RPW) {
    const uint4 v = *reinterpret_cast<const uint4*>(ep + row * S::EPI_ROW + cc * 16);
    const int gm = tok0 + row, gn = ch0 + cc * 8;
    if (gm < M && gn < N)
      *reinterpret_cast<uint4*>(y + static_cast<int64_t>(gm) * ldy + gn) = v;
  }
}

template <int BM, int BN, int BK, int STAGES, int MINB>
hipError_t launch_cfg(const uint8_t* qx, const float* sx, const uint8_t* qw,
                      const float* sw, int64_t m, int64_t n, int64_t k,
                      uint16_t* y, int64_t ldy, hipStream_t stream) {
  const int tiles_m = static_cast<int>((m + BM - 1) / BM);
  const int tiles_n = static_cast<int>((n + BN - 1) / BN);
  gemm_fp8_kernel<BM, BN, BK, STAGES, MINB>
      <<<dim3(static_cast<uint32_t>(tiles_m * tiles_n)), dim3(256), 0, stream>>>(
          qx, sx, qw, sw, static_cast<int>(m), static_cast<int>(n),
          static_cast<int>(k), y, ldy, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace detail
using namespace detail;

// Tile configurations; FP8W8A8_GEMM_CONFIG=<index> overrides the choice
// (a tuning aid; every configuration computes the same result).
hipError_t launch_gemm(const uint8_t* qx, const float* sx, const uint8_t* qw,
                       const float* sw, int64_t m, int64_t n, int64_t k,
                       uint16_t* y, int64_t ldy, hipStream_t stream) {
  if (m == 0 || n == 0) return hipSuccess;
  int cfg = -1;
  if (const char* e = std::getenv("FP8W8A8_GEMM_CONFIG")) cfg = std::atoi(e);
  if (cfg < 0) {
    // Measured on MI355X for the 4096-token layer shapes: 128x128 tiles with
    // two workgroups per CU are best unless K is long, where the 256x256
    // tile's lower operand traffic per flop wins; narrow outputs (few tiles)
    // prefer the 4-stage 64-byte-K pipeline.
    const int64_t big_tiles = ((m + 255) / 256) * ((n + 255) / 256);
    if (big_tiles < 128) cfg = 2;
    else if (k > 8192 && big_tiles >= 192) cfg = 1;
    else cfg = 3;
  }
  switch (cfg) {
    case 0: return launch_cfg<256, 256, 64, 4, 1>(qx, sx, qw, sw, m, n, k, y, ldy, stream);
    case 1: return launch_cfg<256, 256, 128, 2, 1>(qx, sx, qw, sw, m, n, k, y, ldy, stream);
    case 2: return launch_cfg<128, 128, 64, 4, 2>(qx, sx, qw, sw, m, n, k, y, ldy, stream);
    default: return launch_cfg<128, 128, 128, 2, 2>(qx, sx, qw, sw, m, n, k, y, ldy, stream);
  }
}

}  // namespace fp8w8a8
