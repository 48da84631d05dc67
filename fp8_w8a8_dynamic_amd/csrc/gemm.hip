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
//     in f32, accumulation in f32), with the weight fragment as the A operand
//     so that a lane's accumulators hold one token and runs of consecutive
//     output channels;
//   * a workgroup of WGM x WGN waves owns a BM x BN output tile, each wave a
//     (BM/WGM) x (BN/WGN) sub-tile kept in registers;
//   * K advances 128 bytes per stage.  Stages are copied HBM/L2 -> LDS with
//     buffer_load_dwordx4 ... lds (no trip through VGPRs) into NB (2 or 4)
//     LDS buffers.  Every stage's fragments are read into registers early
//     (the second half of a stage's reads overlaps the previous stage's
//     MFMAs); once all waves hold them a barrier frees the buffer, which is
//     refilled with stage k+NB while the MFMAs run, so NB stages of copies
//     are always in flight, with the copies spread between the MFMAs;
//   * LDS rows are 128 bytes with the 16-byte chunk index XOR-swizzled by
//     ((row >> 1) & 7), so the 16 lanes that the LDS serves together read 16
//     distinct bank groups; the swizzle is applied on the global side (each
//     lane fetches the chunk that belongs at its fixed LDS slot);
//   * workgroup -> tile mapping is XCD-aware: the hardware deals workgroups
//     round-robin over the 8 XCDs, so consecutive logical tiles (which share
//     operand rows in groups of 4 tile-rows) are given to one XCD and its L2;
//   * the epilogue scales, rounds to bf16 and stages the tile in LDS, then
//     writes whole row segments with 16-byte stores;
//   * shapes with few output tiles (a few hundred tokens or less) split K
//     over gridDim.y workgroups per tile; each split stores its raw float32
//     sums and splitk_reduce_kernel adds the splits in order and applies the
//     epilogue (deterministic, no cross-workgroup synchronization).
// Rows beyond M or N read as zero (buffer descriptors bounded to the tile's
// valid rows) and are never stored.  K must be a multiple of 128.
#include <cstdlib>
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace fp8w8a8 {

namespace detail {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef v4i_t v4i;
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kGroupM = 4;

// s_waitcnt immediate that waits until at most n LDS (and scalar memory)
// operations are outstanding (gfx9 encoding; vmcnt and expcnt left at their
// maxima).
constexpr int lgkmcnt_imm(int n) { return 15 | (3 << 14) | (7 << 4) | ((n & 15) << 8); }
constexpr int kBK = 128;     // K bytes per stage

// Tile configuration: BM x BN output tile per workgroup of WGM x WGN waves,
// NB stage buffers in LDS (stages in flight).
template <int BM, int BN, int WGM, int WGN, int NB>
struct GemmShape {
  static constexpr int WAVES = WGM * WGN;
  static constexpr int WM = BM / WGM, WN = BN / WGN;  // wave tile
  static constexpr int TM = WM / 32, TN = WN / 32;  // 32x32 MFMA tiles
  static constexpr int CH = kBK / 16;               // 16-byte chunks per row
  static constexpr int RPI = 1024 / kBK;            // rows per 1 KB copy
  static constexpr int A_STAGE = BM * kBK, B_STAGE = BN * kBK;
  static constexpr int STAGE = A_STAGE + B_STAGE;
  static constexpr int LDS = NB * STAGE;
  static_assert(NB == 2 || NB == 4, "two or four stage buffers");
  static constexpr int A_LOADS = A_STAGE / (1024 * WAVES);  // 1 KB copies
  static constexpr int B_LOADS = B_STAGE / (1024 * WAVES);  // per wave
  static constexpr int COPIES = A_LOADS + B_LOADS;          // per stage
  // Epilogue staging: each wave's WM x WN bf16 tile, rows padded by 16 B.
  static constexpr int EPI_ROW = WN * 2 + 16;
  static constexpr int EPI = WAVES * WM * EPI_ROW;
  // The tile's token scales (1 KB) and channel scales (1 KB), copied into
  // LDS at the start so that the epilogue does not wait on global loads.
  static constexpr int SC_OFF = ((LDS > EPI ? LDS : EPI) + 15) / 16 * 16;
  static constexpr int SMEM = SC_OFF + 2048;
  static_assert(BM <= 256 && BN <= 256, "one 1 KB copy per scale vector");
  static_assert(SMEM <= 160 * 1024, "LDS budget of one CU");
  static_assert(A_LOADS >= 1 && B_LOADS >= 1 &&
                A_LOADS * 1024 * WAVES == A_STAGE &&
                B_LOADS * 1024 * WAVES == B_STAGE, "whole 1 KB copies per wave");
  static_assert(TM >= 1 && TN >= 1 && (TM * TN) % 2 == 0, "wave tile");
};

// XOR swizzle of the 16-byte chunk index within a 128-byte row.  gfx950's
// LDS serves a ds_read_b128 16 lanes at a time from 64 four-byte banks (256
// bytes, two rows), and the 16 lanes of a fragment read read 16 consecutive
// rows at the same logical chunk: the swizzle makes their 16 addresses fall
// in 16 distinct 16-byte bank groups.
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

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

// One 32-byte MFMA operand fragment: physical chunks p0 and p0 ^ 1 of a row.
__device__ __forceinline__ v8i lds_frag(const uint8_t* base, int p0) {
  const uint4 lo = *reinterpret_cast<const uint4*>(base + p0 * 16);
  const uint4 hi = *reinterpret_cast<const uint4*>(base + (p0 ^ 1) * 16);
  v8i r;
  r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
  r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
  return r;
}

template <int BM, int BN, int WGM, int WGN, int NB, int MINB>
__global__ __launch_bounds__(64 * WGM * WGN, MINB) void gemm_fp8_kernel(
    const uint8_t* __restrict__ qx, const float* __restrict__ sx,
    const uint8_t* __restrict__ qw, const float* __restrict__ sw, int M,
    int N, int K, uint16_t* __restrict__ y, int64_t ldy, int tiles_m,
    int tiles_n, float* __restrict__ part) {
  using S = GemmShape<BM, BN, WGM, WGN, NB>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[S::SMEM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN, wn = wave % WGN;

  int tm, tn;
  map_tile(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  // Descriptors cover exactly this tile's valid rows.
  const v4i a_rsrc = make_rsrc(qx + static_cast<int64_t>(m0) * K,
                               static_cast<uint32_t>(min(M - m0, BM)) * K);
  const v4i b_rsrc = make_rsrc(qw + static_cast<int64_t>(n0) * K,
                               static_cast<uint32_t>(min(N - n0, BN)) * K);

  // Global -> LDS assignment.  One wave copy fills 1 KB of LDS = RPI rows of
  // 128 bytes; lane j lands at byte 16*j: row j / CH, physical chunk j % CH,
  // which holds logical chunk (j % CH) ^ swz(row).  Copy number q (of the
  // operand's q = wave * LOADS + i) covers rows 8q .. 8q + 7, so its row is
  // 8q + lane / 8 and swz(row) = (4 (q & 1) + lane / 16) & 7: the offset is
  // a lane part that depends only on the parity of q (two registers) plus
  // the wave-uniform 8 q K, which goes with the stage's K into the copy's
  // scalar offset.
  static_assert(S::RPI == 8 && S::CH == 8, "128-byte stage rows");
  uint32_t lane_off[2];
#pragma unroll
  for (int par = 0; par < 2; ++par)
    lane_off[par] = static_cast<uint32_t>((lane / S::CH) * K +
                                          (((lane % S::CH) ^ ((4 * par + (lane >> 4)) & 7)) * 16));
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
  const int fswz = swz(frow);
  const int a_row0 = wm * S::WM + frow;
  const int b_row0 = wn * S::WN + frow;

  // Copy c (0 <= c < COPIES) of the stage starting at K byte k0 into buffer
  // buf.
  auto copy = [&](int c, int buf, uint32_t k0) {
    if (c < S::A_LOADS) {
      const int q = wave * S::A_LOADS + c;
      lds_copy16(a_rsrc, lane_off[q & 1], k0 + static_cast<uint32_t>(8 * q * K),
                 a_lds + buf * S::STAGE + c * 1024);
    } else {
      const int q = wave * S::B_LOADS + (c - S::A_LOADS);
      lds_copy16(b_rsrc, lane_off[q & 1], k0 + static_cast<uint32_t>(8 * q * K),
                 b_lds + buf * S::STAGE + (c - S::A_LOADS) * 1024);
    }
  };

  // K split blockIdx.y of gridDim.y takes stages [kt0, kt0 + KT) (all of
  // K when gridDim.y == 1).
  const int KT_all = K / kBK;
  const int kt0 = static_cast<int>(blockIdx.y) * KT_all / static_cast<int>(gridDim.y);
  const int KT = (static_cast<int>(blockIdx.y) + 1) * KT_all / static_cast<int>(gridDim.y) - kt0;
  const uint32_t kbase = static_cast<uint32_t>(kt0 * kBK);
  // Wave 0 copies the scales first (so the prologue's wait below, which
  // leaves only later stages outstanding, covers them); rows past M or N
  // read as 0.  The split-K partial sums need no scales.
  if (part == nullptr && wave == 0) {
    lds_copy16(make_rsrc(reinterpret_cast<const uint8_t*>(sx + m0),
                         static_cast<uint32_t>(min(M - m0, BM)) * 4u),
               static_cast<uint32_t>(lane) * 16u, 0u, lds0 + S::SC_OFF);
    lds_copy16(make_rsrc(reinterpret_cast<const uint8_t*>(sw + n0),
                         static_cast<uint32_t>(min(N - n0, BN)) * 4u),
               static_cast<uint32_t>(lane) * 16u, 0u, lds0 + S::SC_OFF + 1024);
  }
#pragma unroll
  for (int st = 0; st < NB; ++st)
    if (st < KT) {
#pragma unroll
      for (int c = 0; c < S::COPIES; ++c)
        copy(c, st, kbase + static_cast<uint32_t>(st * kBK));
    }
  // Main loop.  Per stage, each wave runs T MFMAs of step 0 then T of step
  // 1 (T = TM * TN).  A wave drains its LDS reads at roughly 1 KB per 40
  // clocks, so the reads are spread so that no MFMA waits on them:
  //   * the stage's step-1 fragments are read at its start, its step-0
  //     fragments were read during the previous stage;
  //   * after kRel MFMAs (the step-1 reads have landed) a barrier releases the
  //     buffer, and the copies of stage kt+2 into it go out one or two per
  //     MFMA;
  //   * at MFMA kNext (step 0 done, its registers free) the wave waits for
  //     stage kt+1's copies (all but the kBefore newest outstanding), a
  //     barrier makes every wave's copies visible, and the next stage's
  //     step-0 fragments are read under the remaining step-1 MFMAs.
  // kRel and kNext were tuned on MI355X (3/4 and 5/4 of T).
  constexpr int T = S::TM * S::TN;
  constexpr int kMfma = 2 * T;
  constexpr int kRel = T * 12 / 16;
  constexpr int kNext = T * 20 / 16;
  static_assert(kNext >= T && kNext > kRel && kNext < kMfma, "pipeline points");
  constexpr int kSlots = kMfma - kRel;
  constexpr int kPer = (S::COPIES + kSlots - 1) / kSlots;   // copies per MFMA
  constexpr int kBefore =
      (kNext - kRel) * kPer < S::COPIES ? (kNext - kRel) * kPer : S::COPIES;
  const int p0 = (2 * fhalf) ^ fswz, p1 = (4 + 2 * fhalf) ^ fswz;
  v8i af0[S::TM], bf0[S::TN], af1[S::TM], bf1[S::TN];
  // Fragments of one step, in the order the MFMAs consume them.
  auto read_step = [&](v8i* af, v8i* bf, const uint8_t* as, int p) {
    const uint8_t* bs = as + S::A_STAGE;
    af[0] = lds_frag(as + a_row0 * kBK, p);
#pragma unroll
    for (int u = 0; u < S::TN; ++u) bf[u] = lds_frag(bs + (b_row0 + 32 * u) * kBK, p);
#pragma unroll
    for (int t = 1; t < S::TM; ++t) af[t] = lds_frag(as + (a_row0 + 32 * t) * kBK, p);
  };
  // (Waits outside the steady state fall back to "nothing outstanding".)
  if (KT >= NB) __builtin_amdgcn_s_waitcnt(vmcnt_imm((NB - 1) * S::COPIES));
  else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __syncthreads();
  read_step(af0, bf0, smem, p0);
  // One stage.  Whether it refills its buffer (stage kt + NB exists) and
  // whether a next stage follows are compile-time flags: the steady-state
  // loop below has neither branch, so the compiler's wait counts before
  // the step-1 MFMAs only cover the fragments those MFMAs read (behind a
  // branch its count merge was conservative and made them wait for the
  // next stage's fragment reads as well).
  auto stage = [&](int kt, auto refill_c, auto more_c) {
    constexpr bool refill = decltype(refill_c)::value;
    constexpr bool more = decltype(more_c)::value;
    const int buf = kt & (NB - 1);
    // This stage's step-0 fragments (read under the previous stage's last
    // MFMAs) have landed before its step-1 reads go out, so the step-0
    // MFMAs below wait for nothing.
    __builtin_amdgcn_s_waitcnt(lgkmcnt_imm(0));
    read_step(af1, bf1, smem + buf * S::STAGE, p1);
    const uint32_t next_k = kbase + static_cast<uint32_t>((kt + NB) * kBK);
    // Source order is the schedule (reads, MFMAs and copies interleaved as
    // described above): nothing moves across these points.
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < kMfma; ++i) {
      // Every wave holds this stage's fragments: the buffer takes stage
      // kt+NB.
      if (refill && i == kRel) __syncthreads();
      if (more && i == kNext) {
        // Stage kt+1 has landed once only stages kt+2 .. kt+NB-1 and the
        // first kBefore copies of stage kt+NB are outstanding.
        if (refill)
          __builtin_amdgcn_s_waitcnt(vmcnt_imm((NB - 2) * S::COPIES + kBefore));
        else
          __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        __syncthreads();
        read_step(af0, bf0, smem + ((kt + 1) & (NB - 1)) * S::STAGE, p0);
        __builtin_amdgcn_sched_barrier(0);
      }
      const int t = (i / S::TN) % S::TM, u = i % S::TN;
      if (i < T)
        acc[t][u] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            bf0[u], af0[t], acc[t][u], 0, 0, 0, 0, 0, 0);
      else
        acc[t][u] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            bf1[u], af1[t], acc[t][u], 0, 0, 0, 0, 0, 0);
      if (refill && i >= kRel) {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
          const int c = (i - kRel) * kPer + j;
          if (c < S::COPIES) copy(c, buf, next_k);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  using yes = std::integral_constant<bool, true>;
  using no = std::integral_constant<bool, false>;
  int kt = 0;
  for (; kt + NB < KT; ++kt) stage(kt, yes{}, yes{});
  for (; kt + 1 < KT; ++kt) stage(kt, no{}, yes{});
  stage(kt, no{}, no{});

  // Epilogue.  The MFMAs ran with the weight fragment as the A operand, so
  // in the 32x32 accumulator layout a lane holds one token, (lane & 31) of
  // its token tile t, and for each group q = r >> 2 four consecutive output
  // channels 8q + 4*(lane >> 5) + (r & 3) of channel tile u.  Each lane
  // scales its values, packs four bf16 (8 bytes) into this wave's region of
  // LDS laid out [token][channel], and the wave then writes whole rows back
  // with 16-byte stores (coalesced row segments of 2*WN bytes).
  const int tok0 = m0 + wm * S::WM;
  const int ch0 = n0 + wn * S::WN;
  if (part != nullptr) {
    // K split: the raw float32 sums of this split go to part[split][m][n]
    // (16 bytes = 4 consecutive channels per lane and (t, u, q)); the
    // reduction kernel adds the splits in order and applies the scales.
    float* pb = part + static_cast<int64_t>(blockIdx.y) * M * N;
#pragma unroll
    for (int t = 0; t < S::TM; ++t) {
      const int gm = tok0 + 32 * t + frow;
#pragma unroll
      for (int u = 0; u < S::TN; ++u)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int gn = ch0 + 32 * u + 8 * q + 4 * fhalf;
          if (gm < M && gn < N)
            *reinterpret_cast<float4*>(pb + static_cast<int64_t>(gm) * N + gn) =
                make_float4(acc[t][u][4 * q + 0], acc[t][u][4 * q + 1],
                            acc[t][u][4 * q + 2], acc[t][u][4 * q + 3]);
        }
    }
    return;
  }
  __syncthreads();  // every wave is done with the stage buffers
  uint8_t* ep = smem + wave * (S::WM * S::EPI_ROW);
  const float* sc_tok = reinterpret_cast<const float*>(smem + S::SC_OFF) + wm * S::WM;
  const float* sc_ch = reinterpret_cast<const float*>(smem + S::SC_OFF + 1024) + wn * S::WN;
  // Channel scales of this lane: 4 consecutive channels per (u, q).
  float4 ws[S::TN][4];
#pragma unroll
  for (int u = 0; u < S::TN; ++u)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      ws[u][q] = *reinterpret_cast<const float4*>(sc_ch + 32 * u + 8 * q + 4 * fhalf);
#pragma unroll
  for (int t = 0; t < S::TM; ++t) {
    const int tl = 32 * t + frow;                    // token inside the wave tile
    const float xs = sc_tok[tl];
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
  // (When CPR does not divide 64 the last lanes sit out.)
#pragma unroll 4
  for (int row = rr; row < S::WM && lane < RPW * CPR; row += RPW) {
    const uint4 v = *reinterpret_cast<const uint4*>(ep + row * S::EPI_ROW + cc * 16);
    const int gm = tok0 + row, gn = ch0 + cc * 8;
    // The output is written once and not read back by this kernel: the
    // nontemporal hint keeps the burst of a round of tiles finishing
    // together from displacing operand panels in the caches (measured: the
    // 7-Linear prefill step +1.6 %, the packed one +2.6 %).
    if (gm < M && gn < N)
      __builtin_nontemporal_store(
          v4u32_t{v.x, v.y, v.z, v.w},
          reinterpret_cast<v4u32_t*>(y + static_cast<int64_t>(gm) * ldy + gn));
  }
}

// Sum of the K splits in split order, then the epilogue of the unsplit
// kernel: y = bf16_rne(sum * sw[n] * sx[m]).  One thread per 4 consecutive
// channels (n % 16 == 0, so a group never leaves its row).
__global__ __launch_bounds__(256) void splitk_reduce_kernel(
    const float* __restrict__ part, int splits, const float* __restrict__ sx,
    const float* __restrict__ sw, int M, int N, uint16_t* __restrict__ y,
    int64_t ldy) {
  const int64_t groups = static_cast<int64_t>(M) * (N / 4);
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  const int64_t plane = static_cast<int64_t>(M) * N;
  for (int64_t g = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
       g < groups; g += stride) {
    const int m = static_cast<int>(g / (N / 4));
    const int n = static_cast<int>(g - static_cast<int64_t>(m) * (N / 4)) * 4;
    const float* p = part + static_cast<int64_t>(m) * N + n;
    float4 a = *reinterpret_cast<const float4*>(p);
    for (int sp = 1; sp < splits; ++sp) {
      const float4 b = *reinterpret_cast<const float4*>(p + sp * plane);
      a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
    }
    const float4 w = *reinterpret_cast<const float4*>(sw + n);
    const float xs = sx[m];
    uint2 pk;
    pk.x = pack_bf16x2(a.x * w.x * xs, a.y * w.y * xs);
    pk.y = pack_bf16x2(a.z * w.z * xs, a.w * w.w * xs);
    *reinterpret_cast<uint2*>(y + static_cast<int64_t>(m) * ldy + n) = pk;
  }
}

// The same sum and epilogue for one output row per workgroup, followed by
// the per-token quantization of the bf16 row it produced (the next
// Linear's input).  The row is spread over kRqWaves waves so that a row of
// 4096 channels is one 16-byte vector (8 channels) per thread: wave w forms
// the vectors (j * kRqWaves + w) * 64 + lane, j < NV, in registers -- the
// splits added in split order and scaled as above -- and stores them as y;
// then the row's magnitude maximum over those bf16 values (waves meeting
// in LDS) and the quantizer's own device functions.  So y, codes and scale
// are bit for bit those of splitk_reduce_kernel followed by the per-token
// quantizer on y, with one launch and one read of the row fewer.
constexpr int kRqWaves = 8;

template <int NV>
__global__ __launch_bounds__(64 * kRqWaves) void splitk_reduce_quant_kernel(
    const float* __restrict__ part, int splits, const float* __restrict__ sx,
    const float* __restrict__ sw, int M, int N, uint16_t* __restrict__ y,
    int64_t ldy, uint8_t* __restrict__ q, float* __restrict__ scale) {
  __shared__ uint32_t wmax[kRqWaves];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t row = blockIdx.x;
  const int64_t plane = static_cast<int64_t>(M) * N;
  const float* p = part + row * N;
  const float xs = sx[row];
  const auto yr = row_rsrc(y + row * ldy, static_cast<uint32_t>(N) * 2u);
  uint4 v[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int c = ((j * kRqWaves + wave) * 64 + lane) * 8;
    v[j] = make_uint4(0u, 0u, 0u, 0u);
    if (c < N) {
      float4 a = *reinterpret_cast<const float4*>(p + c);
      float4 b = *reinterpret_cast<const float4*>(p + c + 4);
      for (int sp = 1; sp < splits; ++sp) {
        const float4 u = *reinterpret_cast<const float4*>(p + sp * plane + c);
        const float4 t = *reinterpret_cast<const float4*>(p + sp * plane + c + 4);
        a.x += u.x; a.y += u.y; a.z += u.z; a.w += u.w;
        b.x += t.x; b.y += t.y; b.z += t.z; b.w += t.w;
      }
      const float4 wa = *reinterpret_cast<const float4*>(sw + c);
      const float4 wb = *reinterpret_cast<const float4*>(sw + c + 4);
      v[j].x = pack_bf16x2(a.x * wa.x * xs, a.y * wa.y * xs);
      v[j].y = pack_bf16x2(a.z * wa.z * xs, a.w * wa.w * xs);
      v[j].z = pack_bf16x2(b.x * wb.x * xs, b.y * wb.y * xs);
      v[j].w = pack_bf16x2(b.z * wb.z * xs, b.w * wb.w * xs);
      buf_store16(v[j], yr, static_cast<uint32_t>(c) * 2u);
    }
  }
  uint32_t mx = 0;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    mx = pk_max_u16(mx, bf16x2_abs_bits(v[j].x));
    mx = pk_max_u16(mx, bf16x2_abs_bits(v[j].y));
    mx = pk_max_u16(mx, bf16x2_abs_bits(v[j].z));
    mx = pk_max_u16(mx, bf16x2_abs_bits(v[j].w));
  }
  const uint32_t mw = wave_max_u32(max(mx & 0xffffu, mx >> 16));
  if (lane == 0) wmax[wave] = mw;
  __syncthreads();
  uint32_t mrow = wmax[0];
#pragma unroll
  for (int i = 1; i < kRqWaves; ++i) mrow = max(mrow, wmax[i]);
  const float s = row_scale(__uint_as_float(mrow << 16));
  const auto dst = row_rsrc(q + row * N, static_cast<uint32_t>(N));
  quantize_row<NV>(v, make_divisor(s), [&](int j, uint2 cd) {
    buf_store8(cd, dst, ((j * kRqWaves + wave) * 64 + lane) * 8u);
  });
  if (lane == 0 && wave == 0) scale[row] = s;
}

template <int NV>
hipError_t launch_reduce_quant(const float* part, int splits, const float* sx,
                               const float* sw, int64_t m, int64_t n, uint16_t* y,
                               int64_t ldy, uint8_t* q, float* scale, hipStream_t stream) {
  splitk_reduce_quant_kernel<NV>
      <<<dim3(static_cast<uint32_t>(m)), dim3(64 * kRqWaves), 0, stream>>>(
          part, splits, sx, sw, static_cast<int>(m), static_cast<int>(n), y, ldy, q, scale);
  return hipGetLastError();
}

// With splits > 1 the GEMM stores float32 partial sums to `part`; `reduce`
// then launches splitk_reduce_kernel (otherwise the caller reduces them).
template <int BM, int BN, int WGM, int WGN, int NB, int MINB>
hipError_t launch_cfg(const uint8_t* qx, const float* sx, const uint8_t* qw,
                      const float* sw, int64_t m, int64_t n, int64_t k,
                      uint16_t* y, int64_t ldy, int splits, float* part,
                      bool reduce, hipStream_t stream) {
  const int tiles_m = static_cast<int>((m + BM - 1) / BM);
  const int tiles_n = static_cast<int>((n + BN - 1) / BN);
  gemm_fp8_kernel<BM, BN, WGM, WGN, NB, MINB>
      <<<dim3(static_cast<uint32_t>(tiles_m * tiles_n), static_cast<uint32_t>(splits)),
         dim3(64 * WGM * WGN), 0, stream>>>(
          qx, sx, qw, sw, static_cast<int>(m), static_cast<int>(n),
          static_cast<int>(k), y, ldy, tiles_m, tiles_n,
          splits > 1 ? part : nullptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1 || !reduce) return e;
  int64_t blocks = (m * (n / 4) + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  splitk_reduce_kernel<<<dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, stream>>>(
      part, splits, sx, sw, static_cast<int>(m), static_cast<int>(n), y, ldy);
  return hipGetLastError();
}

}  // namespace detail
using namespace detail;

// Tile configuration and K splits.  With the test hooks on (launch.h),
// FP8W8A8_GEMM_CONFIG=<index> overrides the configuration, and with it
// FP8W8A8_GEMM_SPLITS=<n> the number of K splits (1 if unset) -- tuning
// aids; every configuration computes the same result, and the splits
// change only the float32 summation order.
GemmPlan plan_gemm(int64_t m, int64_t n, int64_t k) {
  GemmPlan p{3, 1};
  if (m <= 0 || n <= 0 || k < kBK) return p;
  if (const char* e = test_hook("FP8W8A8_GEMM_CONFIG")) {
    p.cfg = std::atoi(e);
    if (p.cfg >= 0) {
      if (const char* sp = test_hook("FP8W8A8_GEMM_SPLITS")) {
        int v = std::atoi(sp);
        const int kt = static_cast<int>(k / kBK);
        if (v > kt) v = kt;
        if (v > kMaxSplits) v = kMaxSplits;
        p.splits = v < 1 ? 1 : v;
      }
      return p;
    }
  }
  // Measured on MI355X for the 4096-token layer shapes with operands
  // arriving from HBM: 256x256 tiles of eight waves (4x2); narrow outputs
  // (few tiles, one per CU) take 128x128 tiles with four stages in flight,
  // whose pipeline is otherwise bound by the copies' latency.
  const int64_t big_tiles = ((m + 255) / 256) * ((n + 255) / 256);
  p.cfg = big_tiles < 128 ? 4 : 3;
  if (p.cfg == 3) {
    // Whole rounds of one tile per CU (256 CUs): where 256x256 tiles leave a
    // partial last round, 256x192 tiles (0.8 of the time per tile,
    // measured) may fill the rounds better -- e.g. a packed qkv projection,
    // N = 6144: 384 tiles of 256x256 (1.5 rounds) against 512 of 256x192.
    const int64_t tiles8 = ((m + 255) / 256) * ((n + 191) / 192);
    const double t3 = static_cast<double>((big_tiles + 255) / 256);
    const double t8 = 0.8 * static_cast<double>((tiles8 + 255) / 256);
    if (t8 < t3) p.cfg = 8;
  }
  const int64_t tiles4 = ((m + 127) / 128) * ((n + 127) / 128);
  if (p.cfg == 4 && tiles4 > 256) {
    // More than one round of 128x128 tiles (one workgroup per CU) where
    // 256x128 tiles fit in one: e.g. a packed gate|up projection (N = 24576)
    // at 256 tokens, 384 tiles of 128x128 against 192 of 256x128 (measured
    // 48.3 -> 35.5 us).
    const int64_t tiles10 = ((m + 255) / 256) * ((n + 127) / 128);
    if (tiles10 <= 256) p.cfg = 10;
  }
  if (big_tiles < 128 && tiles4 < 128) {
    // Few tokens (m up to a few hundred): too few output tiles to keep the
    // CUs streaming the weights.  128x64 tiles (one workgroup per CU), and
    // K split so that about one workgroup per CU results, at most 8 ways
    // (measured at m = 64 and 256 on the layer's shapes: more splits cost
    // more in partial-sum traffic than they gain); the splits' float32
    // partial sums go through the workspace to a reduction kernel.  (Leaving
    // K = 4096 unsplit looked 20-30 % faster in eager back-to-back calls,
    // where the extra reduction launch costs host time, but made the
    // 36-layer stack replayed as a graph slower: 4.16 -> 4.52 ms per pass at
    // m = 64.)
    p.cfg = 5;
    const int64_t tiles5 = ((m + 127) / 128) * ((n + 63) / 64);
    const int64_t kt = k / kBK;
    int64_t sp = 256 / tiles5;
    if (sp > 8) sp = 8;
    if (sp > kt) sp = kt;
    p.splits = static_cast<int>(sp < 1 ? 1 : sp);
  }
  return p;
}

size_t gemm_partial_bytes(const GemmPlan& p, int64_t m, int64_t n) {
  return p.splits > 1 ? static_cast<size_t>(p.splits) * m * n * sizeof(float) : 0;
}

namespace {

hipError_t gemm_cfg(const GemmPlan& p, const uint8_t* qx, const float* sx,
                    const uint8_t* qw, const float* sw, int64_t m, int64_t n,
                    int64_t k, uint16_t* y, int64_t ldy, float* part, bool reduce,
                    hipStream_t stream) {
  const int sp = p.splits;
  switch (p.cfg) {
    case 0: return launch_cfg<256, 256, 2, 2, 2, 1>(qx, sx, qw, sw, m, n, k, y, ldy, sp, part, reduce, stream);
    case 1: return launch_cfg<256, 256, 2, 4, 2, 1>(qx, sx, qw, sw, m, n, k, y, ldy, sp, part, reduce, stream);
    case 2: return launch_cfg<128, 128, 2, 2, 2, 2>(qx, sx, qw, sw, m, n, k, y, ldy, sp, part, reduce, stream);
    case 3: return launch_cfg<256, 256, 4, 2, 2, 1>(qx, sx, qw, sw, m, n, k, y, ldy, sp, part, reduce, stream);
    case 4: return launch_cfg<128, 128, 2, 2, 4, 1>(qx, sx, qw, sw, m, n, k, y, ldy, sp, part, reduce, stream);
    case 6: return launch_cfg<64, 128, 2, 2, 2, 3>(qx, sx, qw, sw, m, n, k, y, ldy, sp, part, reduce, stream);
    case 7: return launch_cfg<64, 64, 2, 1, 2, 4>(qx, sx, qw, sw, m, n, k, y, ldy, sp, part, reduce, stream);
    case 8: return launch_cfg<256, 192, 4, 2, 2, 1>(qx, sx, qw, sw, m, n, k, y, ldy, sp, part, reduce, stream);
    case 10: return launch_cfg<256, 128, 4, 2, 2, 1>(qx, sx, qw, sw, m, n, k, y, ldy, sp, part, reduce, stream);
    default: return launch_cfg<128, 64, 2, 2, 4, 2>(qx, sx, qw, sw, m, n, k, y, ldy, sp, part, reduce, stream);
  }
}

}  // namespace

hipError_t launch_gemm(const GemmPlan& p, const uint8_t* qx, const float* sx,
                       const uint8_t* qw, const float* sw, int64_t m, int64_t n,
                       int64_t k, uint16_t* y, int64_t ldy, float* part,
                       hipStream_t stream) {
  if (m == 0 || n == 0) return hipSuccess;
  if (p.splits > 1 && part == nullptr) return hipErrorInvalidValue;
  return gemm_cfg(p, qx, sx, qw, sw, m, n, k, y, ldy, part, true, stream);
}

hipError_t launch_gemm_requant(const GemmPlan& p, const uint8_t* qx, const float* sx,
                               const uint8_t* qw, const float* sw, int64_t m, int64_t n,
                               int64_t k, uint16_t* y, int64_t ldy, uint8_t* q,
                               float* scale, float* part, hipStream_t stream) {
  if (m == 0 || n == 0) return hipSuccess;
  if (p.splits > 1 && part == nullptr) return hipErrorInvalidValue;
  if (p.splits == 1 || n > kRequantMaxN || n % 8 != 0) {
    hipError_t e = gemm_cfg(p, qx, sx, qw, sw, m, n, k, y, ldy, part, true, stream);
    return e == hipSuccess ? launch_quant_rows(y, m, n, ldy, q, scale, stream) : e;
  }
  hipError_t e = gemm_cfg(p, qx, sx, qw, sw, m, n, k, y, ldy, part, false, stream);
  if (e != hipSuccess) return e;
  return launch_splitk_reduce_quant(part, p.splits, sx, sw, m, n, y, ldy, q, scale, stream);
}

hipError_t launch_splitk_reduce(const float* part, int splits, const float* sx,
                                const float* sw, int64_t m, int64_t n, uint16_t* y,
                                int64_t ldy, hipStream_t stream) {
  if (m == 0 || n == 0) return hipSuccess;
  if (n % 4 != 0 || splits < 1) return hipErrorInvalidValue;
  int64_t blocks = (m * (n / 4) + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  splitk_reduce_kernel<<<dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, stream>>>(
      part, splits, sx, sw, static_cast<int>(m), static_cast<int>(n), y, ldy);
  return hipGetLastError();
}

hipError_t launch_splitk_reduce_quant(const float* part, int splits, const float* sx,
                                      const float* sw, int64_t m, int64_t n, uint16_t* y,
                                      int64_t ldy, uint8_t* q, float* scale,
                                      hipStream_t stream) {
  if (m == 0 || n == 0) return hipSuccess;
  if (n > kRequantMaxN || n % 8 != 0 || splits < 1) return hipErrorInvalidValue;
  // 512 vectors of 8 channels per j: NV = ceil(n / 4096) <= 4.
  switch ((n + 4095) / 4096) {
    case 1: return launch_reduce_quant<1>(part, splits, sx, sw, m, n, y, ldy, q, scale, stream);
    case 2: return launch_reduce_quant<2>(part, splits, sx, sw, m, n, y, ldy, q, scale, stream);
    case 3: return launch_reduce_quant<3>(part, splits, sx, sw, m, n, y, ldy, q, scale, stream);
    default: return launch_reduce_quant<4>(part, splits, sx, sw, m, n, y, ldy, q, scale, stream);
  }
}

}  // namespace fp8w8a8
