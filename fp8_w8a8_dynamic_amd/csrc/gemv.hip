// Decode-sized FP8_DYNAMIC Linear (1 <= M <= 16 tokens for the K-class
// kernel below, up to 64 for the token-group kernel at the end of the
// file), bound by the HBM bytes of the E4M3 weights (MOSS-VL-Realtime-FP8
// article, section on why the model is quantized: in streaming decode,
// memory bandwidth sets the response speed, and 8-bit weights halve it
// against BF16).
//
// MFMA layout.  Each v_mfma_f32_16x16x128_f8f6f4 multiplies a 16-row A
// operand (weights) by a 16-column B operand (activation codes).  With MP =
// M rounded up to a power of two and C = 16 / MP, the 16 A rows are MP
// weight rows x C "K classes" and the 16 B columns are MP tokens x C
// classes; class c of a row is every C-th 16-byte chunk, so one MFMA (an
// "item") consumes 2 KB of weights: C * 128 contiguous bytes of each of its
// MP rows (M = 1: 2 KB of one row, read by two fully coalesced 1 KB loads).
// Only the accumulator entries whose row class equals the column class are
// partial dot products; their sum over the C classes is the output.  (M = 16
// gives C = 1: the plain 16-row x 16-token tile.)  The matrix cores have
// ample throughput for the discarded entries.
//
// Work decomposition.  MP weight rows form a row group, which is cs items
// long.  A workgroup of 16 waves owns gpw consecutive row groups and deals
// their gpw * cs items to its waves in equal contiguous ranges, so every
// wave streams at most 8 items (16 KB) and the whole workgroup's weights are
// requested at once, before anything else; the grid is about one workgroup
// per CU.  A wave accumulates the items of one row group in its MFMA
// accumulator; a row group that lies wholly inside one wave's range is
// finished by that wave, and one that spans several waves is summed from
// their LDS partials in wave order (deterministic).  No workgroup waits on
// another.
//
// Activations.  The workgroup stages the activation codes in LDS: in fused
// mode (bf16 in) it loads the rows into registers before issuing the weight
// loads (so they arrive first), takes each row's amax (integer max on bf16
// bits), derives the float32 scale and quantizes into LDS with exactly the
// arithmetic of the stand-alone quantization kernel, all while the weights
// are in flight; unfused, it copies the codes.  Shapes whose codes do not
// fit read them from global memory instead.  Two more fused modes put the
// BF16 step in front of the quantization into the staging: the RMSNorm
// (x and gamma; the row sums in the block order of row_ops.h, through LDS)
// and the SiLU-gated activation (gate and up), each with the arithmetic of
// its stand-alone kernel, so the codes are those the two-step path makes.
#include <algorithm>
#include <cstdlib>

#include "device_common.h"
#include "launch.h"
#include "row_ops.h"

namespace fp8w8a8 {

namespace detail {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 16;
constexpr int kThreads = kWaves * 64;
constexpr int kItems = 8;              // items in flight per wave
constexpr int kLdsRowPad = 16;         // LDS code rows: K + 16 bytes
constexpr int64_t kStageLds = 80 * 1024;  // + 48 KB of partials
constexpr int64_t kFusedElems = 16384;  // in-kernel quantization up to M*K
constexpr int kFusedRegs = kFusedElems / 8 / kThreads;  // x loads per thread
constexpr int kMaxNormBlocksPerRow = kFusedElems / 512;  // fused RMSNorm staging

__device__ __forceinline__ v8i to_v8i(uint4 lo, uint4 hi) {
  v8i r;
  r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
  r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
  return r;
}

// Workgroup barrier that orders LDS only.  (__syncthreads also fences
// global memory, which makes every wave wait for all its weight loads in
// flight; the barriers here only publish LDS data.)
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
// Byte offset, within a row, of the 16-byte chunk that lane group g, class
// c, half h of step s covers (C classes; see the header).
__device__ __forceinline__ int chunk_off(int s, int h, int g, int c, int C) {
  return s * (C * 128) + h * (C * 64) + (g * C + c) * 16;
}

// Sum over classes of a 16x16 tile held as [lane][4] (lane = column j +
// 16 * (row >> 2), register = row & 3): output (row rr, token t).  All 16
// candidate reads are issued together (indexes kept in range) and the ones
// past C are dropped.
__device__ __forceinline__ float class_sum(const float (*tile)[4], int rr,
                                           int t, int C) {
  float v[16];
#pragma unroll
  for (int cc = 0; cc < 16; ++cc) {
    const int i = (rr * C + cc) & 15, j = (t * C + cc) & 15;
    v[cc] = tile[j + 16 * (i >> 2)][i & 3];
  }
  float s = 0.0f;
#pragma unroll
  for (int cc = 0; cc < 16; ++cc) s += cc < C ? v[cc] : 0.0f;
  return s;
}

// Sum over the 64 lanes of a wave with DPP moves (no LDS traffic); the
// total lands in lane 63.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL,
                                                    ROW_MASK, 0xf, false));
}
__device__ __forceinline__ float wave_sum_to_63(float v) {
  v += dpp_f<0xb1, 0xf>(v);    // quad_perm [1,0,3,2]
  v += dpp_f<0x4e, 0xf>(v);    // quad_perm [2,3,0,1]: quad sums
  v += dpp_f<0x141, 0xf>(v);   // row_half_mirror: 8-lane sums
  v += dpp_f<0x140, 0xf>(v);   // row_mirror: 16-lane (row) sums
  v += dpp_f<0x142, 0xa>(v);   // row_bcast:15 into rows 1 and 3
  v += dpp_f<0x143, 0xc>(v);   // row_bcast:31 into rows 2 and 3
  return v;
}

// STAGE: 0 = codes read from global memory, 1 = codes copied to LDS,
// 2 = bf16 activations quantized into LDS (fused), 3 = RMSNorm of x with
// weight x2 (eps) then quantized (needs K % 512 == 0), 4 = SiLU-gated
// activation of gate x and up x2 (row stride ld2) then quantized.  XR: activation loads per
// thread for staging.  NI: weight items loaded per wave and batch; every
// wave issues exactly 2 * NI weight loads per batch (items past its range
// re-read its last item), so that the wait counts before each use are
// static and every MFMA starts as soon as its own item has landed.
template <int STAGE, int XR, int NI>
__global__ __launch_bounds__(kThreads) void gemv_fp8_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, const uint8_t* __restrict__ qx,
    const float* __restrict__ sx, const uint8_t* __restrict__ qw,
    const float* __restrict__ sw, int M, int lg_mp, int N, int K, int gpw,
    uint16_t* __restrict__ y, int64_t ldy, const uint16_t* __restrict__ x2,
    int64_t ld2, float eps) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds_x[];
  __shared__ float part[kWaves][2][64][4];   // partials of shared row groups
  __shared__ float part1[kWaves][2];         // ... for M = 1 (one value)
  __shared__ float fin[kWaves][64][4];       // per-wave finishing scratch
  __shared__ float s_scale[kGemvMaxM];
  __shared__ uint32_t s_wmax[kWaves][kGemvMaxM];   // per-wave row maxima

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int MP = 1 << lg_mp;
  const int C = 16 >> lg_mp;
  const int cs = (K + C * 128 - 1) / (C * 128);  // items per row group
  const int g0 = blockIdx.x * gpw;               // first row group
  const int gcount = min(gpw, (N >> lg_mp) - g0);
  const int total = gcount * cs;
  const int a = (wave * total) / kWaves, b = ((wave + 1) * total) / kWaves;

  const int i16 = lane & 15, g = lane >> 4;
  const int r = i16 / C, c = i16 % C;            // A: weight row, class
  const int tok = i16 / C;                       // B: token (same class c)
  const bool tok_ok = tok < M;
  // LDS code rows: K + 16 bytes; copied rows (STAGE 1) are padded to whole
  // 1 KB copies first.
  const int lds_stride = (STAGE == 1 ? (K + 1023) / 1024 * 1024 : K) + kLdsRowPad;

  // 1) Staging loads of the activations, issued first.
  uint4 xv[STAGE >= 2 ? XR : 1];
  uint4 x2v[STAGE >= 3 ? XR : 1];
  uint32_t after = 0;   // produced after the staging loads (see below)
  if constexpr (STAGE >= 2) {
    const int kv8 = K / 8;
#pragma unroll
    for (int i = 0; i < XR; ++i) {
      // Clamped index: every lane loads (a valid address); only in-range
      // elements are used.
      const int e = min(tid + i * kThreads, M * kv8 - 1);
      const int m = e / kv8, v = e - m * kv8;
      xv[i] = *reinterpret_cast<const uint4*>(x + m * ldx + v * 8);
      if constexpr (STAGE == 3)
        x2v[i] = *reinterpret_cast<const uint4*>(x2 + v * 8);          // gamma
      else if constexpr (STAGE == 4)
        x2v[i] = *reinterpret_cast<const uint4*>(x2 + m * ld2 + v * 8);  // up
    }
    // Each wave clears its own row maxima (wave-private: no barrier).
    if (lane < kGemvMaxM) s_wmax[wave][lane] = 0u;
  } else if constexpr (STAGE == 1) {
    // 1 KB copies of the code rows straight into LDS, dealt to the waves.
    // Lanes past a row's end copy the next row's first bytes into this
    // row's padding (never read); past the last row the descriptor reads 0.
    const v4i_t rs = make_rsrc(qx, static_cast<uint32_t>(M * K));
    const int nch = (K + 1023) / 1024;
    const uint32_t l0 = __builtin_amdgcn_readfirstlane(lds_addr(lds_x));
    for (int q = wave; q < M * nch; q += kWaves) {
      const int m = q / nch, ch = q - m * nch;
      lds_copy16(rs, static_cast<uint32_t>(m * K + ch * 1024 + lane * 16), 0u,
                 l0 + m * lds_stride + ch * 1024);
    }
  }
  // The weight addresses below take `after`, written by an asm statement
  // that follows the staging loads: the weight loads cannot be issued before
  // them, so waiting for "2 * NI outstanding" covers every staging load.
  asm volatile("s_mov_b32 %0, 0" : "=s"(after) : : "memory");

  // 2) Weight loads of this wave's first NI items.  Item it is step
  // (it % cs) of row group (it / cs).  The first kEarly items go out now;
  // the rest after the activation codes are staged, so that every wave
  // reaches the staging barriers quickly (a wave blocks while the memory
  // pipeline is full, and kEarly items per wave keep it full meanwhile).
  constexpr int kEarly = NI < 2 ? NI : 2;
  uint4 wa[NI][2];
  const int last = b > a ? b - 1 : min(a, total - 1);
  auto load_item = [&](int s, int first, uint32_t dep) {
    const int it = min(first + s, last);
    const int gl = it / cs, st = it - gl * cs;
    const uint8_t* rp =
        qw + static_cast<int64_t>((g0 + gl) * MP + r) * K + dep;
    // Chunks past K (a partial last step) re-read the row's last chunk:
    // their B operand is zero, so they add nothing.  The loads carry no
    // condition, which keeps their number, and the waits, static.
#pragma unroll
    for (int h = 0; h < 2; ++h)
      wa[s][h] = load16_stream(rp + min(chunk_off(st, h, g, c, C), K - 16));
  };
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int s = 0; s < kEarly; ++s) load_item(s, a, after);
  // A use of the loaded registers on a path never taken (K > 0): the loads
  // must stay here, ahead of the barriers below, instead of being sunk to
  // their MFMAs.  It costs one scalar compare and forces no wait on the
  // path taken.
  if (K <= 0) {
    uint32_t z = 0;
#pragma unroll
    for (int s = 0; s < kEarly; ++s) z ^= wa[s][0].x ^ wa[s][1].x;
    y[0] = static_cast<uint16_t>(z);
  }
  __builtin_amdgcn_sched_barrier(0);

  // 3) Activation codes into LDS.
  if constexpr (STAGE == 4) {
    // h = bf16(bf16(silu(gate)) * up) in place; the silu form is chosen per
    // wave slot, which changes no result (row_ops.h).
    const int kv8 = K / 8;
#pragma unroll
    for (int i = 0; i < XR; ++i) {
      const int e0 = i * kThreads + wave * 64;
      if (e0 < M * kv8) {
        const bool ok = e0 + lane < M * kv8;
        float unused = 0.0f;
        xv[i] = __builtin_amdgcn_ballot_w64(ok && any_deep8(xv[i])) == 0
                    ? swiglu8<true>(xv[i], x2v[i], unused)
                    : swiglu8<false>(xv[i], x2v[i], unused);
      }
    }
  } else if constexpr (STAGE == 3) {
    // y = bf16(gamma * bf16(x / sqrt(mean(x^2) + eps))) in place.  With
    // K % 512 == 0 a wave slot is one whole 512-value block of one row: its
    // sum is block_sumsq, and the blocks of a row are added in order after
    // one barrier, exactly as the stand-alone norm kernel adds them.
    __shared__ float s_blk[kGemvMaxM][kMaxNormBlocksPerRow];
    __shared__ float s_blk2[kGemvMaxM][kMaxNormBlocksPerRow];
    __shared__ uint32_t s_amx[kWaves][kGemvMaxM];
    const int kv8 = K / 8, nblk = kv8 / 64;
#pragma unroll
    for (int i = 0; i < XR; ++i) {
      const int e0 = i * kThreads + wave * 64;
      if (e0 < M * kv8) {
        const int m = e0 / kv8, b = (e0 - m * kv8) / 64;
        const float bs = block_sumsq(xv[i]);
        if (lane == 0) s_blk[m][b] = bs;
      }
    }
    if (lane < kGemvMaxM) s_amx[wave][lane] = 0u;
    lds_barrier();
    auto row_ss = [&](const float (*blk)[kMaxNormBlocksPerRow], int m) {
      float ss = 0.0f;
      for (int b = 0; b < nblk; ++b) ss += blk[m][b];
      return ss;
    };
    bool rare_any = false;                       // uniform: every thread reads
    for (int m = 0; m < M; ++m) rare_any |= !sumsq_in_range(row_ss(s_blk, m));
    if (rare_any) {
      // The rare, exactly scaled path (rows whose float32 sum of squares
      // under- or overflows): p from the row's amax, then the scaled sums.
#pragma unroll
      for (int i = 0; i < XR; ++i) {
        const int e0 = i * kThreads + wave * 64;
        if (e0 < M * kv8) {
          const uint32_t mm = amax8_bits(xv[i], 0u);
          const uint32_t wm = wave_max_u32(max(mm & 0xffffu, mm >> 16));
          if (lane == 0) s_amx[wave][e0 / kv8] = max(s_amx[wave][e0 / kv8], wm);
        }
      }
      lds_barrier();
#pragma unroll
      for (int i = 0; i < XR; ++i) {
        const int e0 = i * kThreads + wave * 64;
        if (e0 < M * kv8) {
          const int m = e0 / kv8, b = (e0 - m * kv8) / 64;
          uint32_t am = 0;
          for (int w = 0; w < kWaves; ++w) am = max(am, s_amx[w][m]);
          const float bs = block_sumsq_scaled(xv[i], pow2_for_amax(am));
          if (lane == 0) s_blk2[m][b] = bs;
        }
      }
      lds_barrier();
    }
#pragma unroll
    for (int i = 0; i < XR; ++i) {
      const int e0 = i * kThreads + wave * 64;
      if (e0 < M * kv8) {
        const int m = e0 / kv8;
        float ss = row_ss(s_blk, m), p = 1.0f;
        if (!sumsq_in_range(ss)) {
          uint32_t am = 0;
          for (int w = 0; w < kWaves; ++w) am = max(am, s_amx[w][m]);
          p = pow2_for_amax(am);
          ss = row_ss(s_blk2, m);
        }
        float unused = 0.0f;
        xv[i] = norm8(xv[i], x2v[i], make_norm_factor(ss, K, eps, p), unused);
      }
    }
  }
  if constexpr (STAGE >= 2) {
    // Row amax (integer max on bf16 magnitude bits): each wave into its own
    // slots, then one barrier, after which every thread takes the max over
    // the waves for the rows it quantizes.
    const int kv8 = K / 8;
#pragma unroll
    for (int i = 0; i < XR; ++i) {
      const int e0 = i * kThreads + wave * 64;   // first element of the wave
      if (e0 < M * kv8) {
        const int e = e0 + lane;
        const bool ok = e < M * kv8;
        uint32_t mm = 0;
        if (ok) {
          mm = pk_max_u16(bf16x2_abs_bits(xv[i].x), bf16x2_abs_bits(xv[i].y));
          mm = pk_max_u16(mm, bf16x2_abs_bits(xv[i].z));
          mm = pk_max_u16(mm, bf16x2_abs_bits(xv[i].w));
          mm = max(mm & 0xffffu, mm >> 16);
        }
        const int m_first = e0 / kv8;
        const int m_last = min(e0 + 63, M * kv8 - 1) / kv8;
        if (m_first == m_last) {
          const uint32_t wm = wave_max_u32(mm);
          if (lane == 0) s_wmax[wave][m_first] = max(s_wmax[wave][m_first], wm);
        } else if (ok) {
          atomicMax(&s_wmax[wave][e / kv8], mm);
        }
      }
    }
    lds_barrier();
    auto scale_row = [&](int m) {
      uint32_t am = 0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) am = max(am, s_wmax[w][m]);
      return row_scale(__uint_as_float(am << 16));
    };
    if (tid < M) s_scale[tid] = scale_row(tid);   // for the epilogue
#pragma unroll
    for (int i = 0; i < XR; ++i) {
      const int e = tid + i * kThreads;
      if (e < M * kv8) {
        const int m = e / kv8, v = e - m * kv8;
        *reinterpret_cast<uint2*>(lds_x + m * lds_stride + v * 8) =
            quantize8(xv[i], make_divisor(scale_row(m)));
      }
    }
    lds_barrier();
  } else if constexpr (STAGE == 1) {
    // This wave's copies are older than its 2 * kEarly weight loads.
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * kEarly));
    lds_barrier();
  }

  // The remaining items of the first batch; their addresses depend on an
  // asm statement after the staging barriers, so they cannot be hoisted
  // above them (nor above the manual wait of the LDS copies).
  if constexpr (NI > kEarly) {
    uint32_t after2;
    asm volatile("s_mov_b32 %0, 0" : "=s"(after2) : : "memory");
#pragma unroll
    for (int s = kEarly; s < NI; ++s) load_item(s, a, after2);
  }

  // B fragment of step st (zero for tokens >= M and for chunks past K).
  auto load_b = [&](int st) -> v8i {
    uint4 hv[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int off = chunk_off(st, h, g, c, C);
      const bool ok = tok_ok && off < K;
      const int o = ok ? off : 0;
      const int t = tok_ok ? tok : 0;
      uint4 v;
      if constexpr (STAGE == 0)
        v = *reinterpret_cast<const uint4*>(qx + static_cast<int64_t>(t) * K + o);
      else
        v = *reinterpret_cast<const uint4*>(lds_x + t * lds_stride + o);
      hv[h] = ok ? v : make_uint4(0u, 0u, 0u, 0u);
    }
    return to_v8i(hv[0], hv[1]);
  };

  auto scale_of = [&](int t) { return STAGE >= 2 ? s_scale[t] : sx[t]; };
  const int outs = MP * M;   // outputs of one row group

  // A row group is done with this wave's contribution: finish it here if it
  // lies wholly inside [a, b), else leave the partial for the workgroup.
  const int g_first = a / cs;
  auto flush = [&](int gl, const v4f& acc) {
    const bool inside = gl * cs >= a && (gl + 1) * cs <= b;
    if (C == 16) {
      // M = 1: the output is the sum of the diagonal, which lane l holds in
      // register (l & 15) - 4 * (l >> 4) when that is in 0..3.
      const int qd = (lane & 15) - 4 * (lane >> 4);
      float d = qd == 0 ? acc[0] : qd == 1 ? acc[1] : qd == 2 ? acc[2]
              : qd == 3 ? acc[3] : 0.0f;
      d = wave_sum_to_63(d);
      if (lane == 63) {
        if (inside) {
          const int n = g0 + gl;
          y[n] = f32_to_bf16_bits(d * sw[n] * scale_of(0));
        } else {
          part1[wave][gl == g_first ? 0 : 1] = d;
        }
      }
      return;
    }
    if (inside) {
#pragma unroll
      for (int q = 0; q < 4; ++q) fin[wave][lane][q] = acc[q];
      __builtin_amdgcn_wave_barrier();
      for (int o = lane; o < outs; o += 64) {
        const int rr = o % MP, t = o / MP;
        const int n = (g0 + gl) * MP + rr;
        const float v = class_sum(fin[wave], rr, t, C);
        y[static_cast<int64_t>(t) * ldy + n] =
            f32_to_bf16_bits(v * sw[n] * scale_of(t));
      }
      __builtin_amdgcn_wave_barrier();
    } else {
      const int si = gl == g_first ? 0 : 1;
#pragma unroll
      for (int q = 0; q < 4; ++q) part[wave][si][lane][q] = acc[q];
    }
  };

  // 4) The items: one MFMA each, row group by row group (the accumulator is
  // flushed where a row group or this wave's range ends).  More than NI
  // items per wave (a row group longer than the workgroup can hold) are
  // loaded batch by batch.
  v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
  auto run_batch = [&](int base) {             // items [base, base + nb)
    const int nb = min(NI, b - base);
    int s0 = 0;
    while (s0 < nb) {
      const int gl = (base + s0) / cs;
      const int s1 = min(nb, (gl + 1) * cs - base);   // end of the group here
      const int st0 = base - gl * cs;                 // step of slot 0
#pragma unroll
      for (int s = 0; s < NI; ++s)
        if (s >= s0 && s < s1)
          acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              to_v8i(wa[s][0], wa[s][1]), load_b(st0 + s), acc,
              0, 0, 0, 0, 0, 0);
      if (base + s1 == (gl + 1) * cs || base + s1 == b) {
        flush(gl, acc);
        acc = v4f{0.0f, 0.0f, 0.0f, 0.0f};
      }
      s0 = s1;
    }
  };
  // The first batch in straight-line code (its loads are the ones issued
  // above), later batches in a loop.
  if (a < b) run_batch(a);
  for (int base = a + NI; base < b; base += NI) {
#pragma unroll
    for (int s = 0; s < NI; ++s) load_item(s, base, 0u);
    run_batch(base);
  }

  // 5) Row groups shared by several waves: sum the partials in wave order.
  lds_barrier();
  for (int o = tid; o < gcount * outs; o += kThreads) {
    const int gl = o / outs, rr = o % MP, t = (o % outs) / MP;
    const int lo = gl * cs, hi = lo + cs;
    // Waves whose (non-empty) ranges meet the group: w_lo .. w_hi.
    int w_lo = kWaves, w_hi = -1;
    for (int w = 0; w < kWaves; ++w) {
      const int aw = (w * total) / kWaves, bw = ((w + 1) * total) / kWaves;
      if (aw < bw && aw < hi && bw > lo) {
        w_lo = min(w_lo, w);
        w_hi = w;
      }
    }
    if (w_hi > w_lo) {
      float v = 0.0f;
      for (int w = w_lo; w <= w_hi; ++w) {
        const int aw = (w * total) / kWaves, bw = ((w + 1) * total) / kWaves;
        if (aw < bw) {
          const int si = gl == aw / cs ? 0 : 1;
          v += C == 16 ? part1[w][si] : class_sum(part[w][si], rr, t, C);
        }
      }
      const int n = (g0 + gl) * MP + rr;
      y[static_cast<int64_t>(t) * ldy + n] = f32_to_bf16_bits(v * sw[n] * scale_of(t));
    }
  }
}

// Token-group GEMV for 16 < M <= 64 (T = ceil(M / 16) groups of 16 tokens):
// the same v_mfma_f32_16x16x128_f8f6f4 with one K class (the A operand is 16
// weight rows x 128 K bytes, the B operand 16 tokens x the same 128 bytes),
// each weight fragment feeding T MFMAs.  A 4-wave workgroup owns 16 weight
// rows (one row group) over all of K; the waves split K four ways, load
// weights and activation codes straight into registers (the codes of one
// K range are read by one wave only, so LDS staging would buy nothing) in
// batches of kTokBatch items with the next batch in flight, and add their
// sums in LDS in wave order.  One kernel, no workspace partial sums.
constexpr int kTokWaves = 4;

template <int T>
__global__ __launch_bounds__(kTokWaves * 64) void gemv_tok_kernel(
    const uint8_t* __restrict__ qx, const float* __restrict__ sx,
    const uint8_t* __restrict__ qw, const float* __restrict__ sw, int M,
    int K, uint16_t* __restrict__ y, int64_t ldy) {
  constexpr int kB = T <= 2 ? 4 : 2;                // items per batch
  __shared__ float red[kTokWaves][T][64][4];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n0 = blockIdx.x * 16;
  const int r = lane & 15, g = lane >> 4;
  const int ks = K / 128;                           // items of the row group
  const int s0 = wave * ks / kTokWaves, s1 = (wave + 1) * ks / kTokWaves;
  // Lane (r, g) holds bytes g*16 .. +15 and 64 + g*16 .. +15 of each
  // 128-byte step, for weight row n0 + r and for token 16 t + r: the same
  // K order on both operands.
  const uint8_t* wrow = qw + static_cast<int64_t>(n0 + r) * K + g * 16;
  const uint8_t* xrow[T];
  bool tok_ok[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int tok = 16 * t + r;
    tok_ok[t] = tok < M;
    xrow[t] = qx + static_cast<int64_t>(tok_ok[t] ? tok : 0) * K + g * 16;
  }
  v4f acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  uint4 wa[2][kB][2], xb[2][kB][T][2];
  // Items past the wave's range re-read its last item (a static number of
  // loads); their MFMAs are skipped.
  auto load = [&](int buf, int s) {
#pragma unroll
    for (int i = 0; i < kB; ++i) {
      const int si = min(s + i, s1 - 1) * 128;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        wa[buf][i][h] = load16_stream(wrow + si + h * 64);
#pragma unroll
        for (int t = 0; t < T; ++t)
          xb[buf][i][t][h] = *reinterpret_cast<const uint4*>(xrow[t] + si + h * 64);
      }
    }
  };
  auto run = [&](int buf, int s) {
#pragma unroll
    for (int i = 0; i < kB; ++i)
      if (s + i < s1) {
        const v8i a = to_v8i(wa[buf][i][0], wa[buf][i][1]);
#pragma unroll
        for (int t = 0; t < T; ++t) {
          const v8i b = tok_ok[t] ? to_v8i(xb[buf][i][t][0], xb[buf][i][t][1])
                                  : v8i{0, 0, 0, 0, 0, 0, 0, 0};
          acc[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              a, b, acc[t], 0, 0, 0, 0, 0, 0);
        }
      }
  };
  if (s0 < s1) {
    load(0, s0);
    for (int s = s0; s < s1; s += 2 * kB) {
      if (s + kB < s1) load(1, s + kB);
      run(0, s);
      if (s + kB < s1) {
        if (s + 2 * kB < s1) load(0, s + 2 * kB);
        run(1, s + kB);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int q = 0; q < 4; ++q) red[wave][t][lane][q] = acc[t][q];
  __syncthreads();
  // Lane l's accumulator q is the dot product of weight row 4 (l >> 4) + q
  // and token l & 15 of its group: 4 consecutive outputs of one token.
  for (int o = tid; o < T * 64; o += kTokWaves * 64) {
    const int t = o / 64, l = o % 64;
    const int tok = 16 * t + (l & 15);
    if (tok < M) {
      const int n = n0 + 4 * (l >> 4);
      const float xs = sx[tok];
      float v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float a = red[0][t][l][q];
#pragma unroll
        for (int w = 1; w < kTokWaves; ++w) a += red[w][t][l][q];
        v[q] = a * sw[n + q] * xs;
      }
      uint2 pk;
      pk.x = pack_bf16x2(v[0], v[1]);
      pk.y = pack_bf16x2(v[2], v[3]);
      *reinterpret_cast<uint2*>(y + static_cast<int64_t>(tok) * ldy + n) = pk;
    }
  }
}

}  // namespace detail
using namespace detail;

hipError_t launch_gemv_tok(const uint8_t* qx, const float* sx,
                           const uint8_t* qw, const float* sw, int64_t m,
                           int64_t n, int64_t k, uint16_t* y, int64_t ldy,
                           hipStream_t stream) {
  if (m == 0 || n == 0) return hipSuccess;
  if (m > kGemvTokMaxM) return hipErrorInvalidValue;
  const dim3 grid(static_cast<uint32_t>(n / 16)), block(kTokWaves * 64);
  const int mi = static_cast<int>(m), ki = static_cast<int>(k);
  switch ((m + 15) / 16) {
    case 1: gemv_tok_kernel<1><<<grid, block, 0, stream>>>(qx, sx, qw, sw, mi, ki, y, ldy); break;
    case 2: gemv_tok_kernel<2><<<grid, block, 0, stream>>>(qx, sx, qw, sw, mi, ki, y, ldy); break;
    case 3: gemv_tok_kernel<3><<<grid, block, 0, stream>>>(qx, sx, qw, sw, mi, ki, y, ldy); break;
    default: gemv_tok_kernel<4><<<grid, block, 0, stream>>>(qx, sx, qw, sw, mi, ki, y, ldy); break;
  }
  return hipGetLastError();
}

// Fused (in-kernel) quantization pays for re-quantizing the activations in
// every workgroup; measured on MI355X it beats a separate quantization
// kernel up to about 16K activation elements.
bool gemv_fused_fits(int64_t m, int64_t n, int64_t k) {
  (void)n;
  return m * k <= kFusedElems &&
         m * (k / 8) <= static_cast<int64_t>(kFusedRegs) * kThreads &&
         m * (k + kLdsRowPad) <= kStageLds;
}

// The fused pre-step's extra operand: gamma and eps (STAGE 3) or up (STAGE 4).
struct GemvPre {
  const uint16_t* x2;
  int64_t ld2;
  float eps;
};

template <int STAGE, int XR, int NI>
hipError_t launch_ni(const uint16_t* x, int64_t ldx, const uint8_t* qx,
                     const float* sx, const uint8_t* qw, const float* sw,
                     int64_t m, int lg_mp, int64_t n, int64_t k, int gpw,
                     uint16_t* y, int64_t ldy, const GemvPre& pre,
                     hipStream_t stream) {
  const int64_t groups = n >> lg_mp;
  const dim3 grid(static_cast<uint32_t>((groups + gpw - 1) / gpw));
  const size_t lds = STAGE == 0 ? 0
                   : static_cast<size_t>(m) *
                         ((STAGE == 1 ? (k + 1023) / 1024 * 1024 : k) + kLdsRowPad);
  gemv_fp8_kernel<STAGE, XR, NI><<<grid, dim3(kThreads), lds, stream>>>(
      x, ldx, qx, sx, qw, sw, static_cast<int>(m), lg_mp, static_cast<int>(n),
      static_cast<int>(k), gpw, y, ldy, pre.x2, pre.ld2, pre.eps);
  return hipGetLastError();
}

template <int STAGE, int XR>
hipError_t launch_one(const uint16_t* x, int64_t ldx, const uint8_t* qx,
                      const float* sx, const uint8_t* qw, const float* sw,
                      int64_t m, int lg_mp, int64_t n, int64_t k, int gpw,
                      int ni, uint16_t* y, int64_t ldy, const GemvPre& pre,
                      hipStream_t stream) {
#define FP8W8A8_GEMV_NI(NI) \
  return launch_ni<STAGE, XR, NI>(x, ldx, qx, sx, qw, sw, m, lg_mp, n, k, gpw, y, ldy, pre, stream)
  switch (ni) {
    case 1: FP8W8A8_GEMV_NI(1);
    case 2: FP8W8A8_GEMV_NI(2);
    case 3: FP8W8A8_GEMV_NI(3);
    case 4: FP8W8A8_GEMV_NI(4);
    case 6: FP8W8A8_GEMV_NI(6);
    default: FP8W8A8_GEMV_NI(8);
  }
#undef FP8W8A8_GEMV_NI
}

struct GemvPlan {
  int lg_mp, gpw, ni;
};

GemvPlan plan_gemv(int64_t m, int64_t n, int64_t k) {
  int lg_mp = 0;
  while ((1 << lg_mp) < m) ++lg_mp;
  // Row groups per workgroup, measured on MI355X at M = 1, 2, 4, 8 on the
  // layer's shapes.  The workgroup count aims at one per CU but no fewer
  // than ~64 KB of weights per workgroup (64 to 256 workgroups): every
  // workgroup pays for staging the activations, so small matrices (k/v,
  // 4 MB) stream fastest from 64 workgroups, and e.g. q at M = 4 from 256
  // rather than 64 (12.1 -> 9.9 us).  Where a workgroup holds at least one
  // row group per wave and the groups fit one batch of loads, they are
  // dealt whole to the waves (none shared); where one workgroup per CU
  // would then need more groups per wave than a batch holds, the groups are
  // split evenly over 2, 3, ... workgroups per CU (a count that leaves some
  // CUs one workgroup more than others costs a whole extra workgroup time:
  // 24576 x 4096 took 27.4 us with 384 workgroups, 22.5 us with 512).
  // Otherwise groups are shared between waves, up to one batch per wave.
  const int64_t groups = n >> lg_mp;
  const int64_t cs = (k + (2048 >> lg_mp) - 1) / (2048 >> lg_mp);
  int64_t wgs = n * k / 65536;
  if (wgs > 256) wgs = 256;
  if (wgs < 64) wgs = 64;
  int64_t gpw = (groups + wgs - 1) / wgs;
  // Share of the last round of one workgroup per CU that is filled.
  auto filled = [&](int64_t g) {
    const int64_t c = (groups + g - 1) / g;
    return c <= 256 ? 1.0 : static_cast<double>(c) / (256.0 * ((c + 255) / 256));
  };
  // Largest of unit, 2 unit, ... top with the fullest last round.
  auto best_fill = [&](int64_t unit, int64_t top) {
    int64_t pick = unit;
    for (int64_t g = unit; g <= top; g += unit)
      if (filled(g) >= filled(pick)) pick = g;
    return pick;
  };
  const int64_t cap = (kWaves * kItems) / cs;   // one batch per wave
  if (cs <= kItems && gpw >= kWaves) {
    const int64_t need = (gpw + kWaves - 1) / kWaves;
    const int64_t fit = kItems / cs;
    gpw = need <= fit ? kWaves * need : best_fill(kWaves, kWaves * fit);
    if (filled(gpw) < 1.0) {
      const int64_t shared = best_fill(1, cap);
      if (filled(shared) > filled(gpw)) gpw = shared;
    }
  } else {
    if (gpw > cap) gpw = best_fill(1, cap);
    if (gpw < 1) gpw = 1;
  }
  // With the test hooks on, FP8W8A8_GEMV_GPW overrides (a tuning aid; every choice computes the
  // same result up to float32 summation order).
  if (const char* e = test_hook("FP8W8A8_GEMV_GPW")) {
    const int64_t v = std::atoll(e);
    if (v >= 1 && v <= groups) gpw = v;
  }
  // Items per wave (the most any wave of a full workgroup gets).
  const int64_t per_wave = (gpw * cs + kWaves - 1) / kWaves;
  const int ni = per_wave <= 1 ? 1 : per_wave <= 2 ? 2 : per_wave <= 3 ? 3
               : per_wave <= 4 ? 4 : per_wave <= 6 ? 6 : kItems;
  return GemvPlan{lg_mp, static_cast<int>(gpw), ni};
}

namespace detail {

// One token (M = 1), its quantization fused (or its codes given), without
// LDS or barriers.  At
// M = 1 the K-class layout above gives lane l of step s, half h the 16
// bytes at 2048 s + 1024 h + 16 l of a weight row, and the same 16
// positions of the activation codes.  Every wave owns R whole weight rows
// and therefore needs the codes of the whole row; it loads its own 16-value
// slices of x (the whole row across the wave, each value once), takes the
// row amax with a wave reduction and quantizes in registers with the
// quantizer's own device functions (bit-identical codes).  Per row, the CS
// steps accumulate in order into one MFMA accumulator whose diagonal is
// summed with the DPP tree, then the epilogue: the same order as the
// LDS-staged kernel when it gives a wave whole rows.  The x loads are
// issued before the weight loads, so waiting for them leaves the weights
// in flight; out-of-range bytes (a ragged last step, rows past N) read as 0
// through the buffer descriptors.
// CODES: the activation arrives already quantized (qx, one code per value,
// and its scale sx[0]): the codes are loaded in the same slices instead.
//
// The per-row MFMA chain and its epilogue, shared with the grouped kernel
// below: per row, the CS steps accumulate in order into one accumulator
// whose diagonal (the K-class partial dot products) the DPP tree sums.
template <int CS, int R>
__device__ __forceinline__ void m1_rows_mfma(const uint4 (&wv)[R][CS][2],
                                             const v8i (&bq)[CS], float scale,
                                             const float* __restrict__ sw, int N,
                                             int row0, uint16_t* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int qd = (lane & 15) - 4 * (lane >> 4);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < CS; ++s)
      acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
          to_v8i(wv[r][s][0], wv[r][s][1]), bq[s], acc, 0, 0, 0, 0, 0, 0);
    float dg = qd == 0 ? acc[0] : qd == 1 ? acc[1] : qd == 2 ? acc[2]
             : qd == 3 ? acc[3] : 0.0f;
    dg = wave_sum_to_63(dg);
    const int n = row0 + r;
    if (lane == 63 && n < N) y[n] = f32_to_bf16_bits(dg * sw[n] * scale);
  }
}

// The whole body of gemv_m1_kernel for the wave whose first row is row0.
template <int CS, int R, bool CODES>
__device__ __forceinline__ void m1_rows(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ qx,
    const float* __restrict__ sx, const uint8_t* __restrict__ qw,
    const float* __restrict__ sw, int N, int K, uint16_t* __restrict__ y,
    int row0) {
  const int lane = threadIdx.x & 63;
  uint4 xv[CODES ? 1 : CS][2][2];
  uint4 cv[CODES ? CS : 1][2];
  if constexpr (CODES) {
    const auto csrc = row_rsrc(qx, static_cast<uint32_t>(K));
#pragma unroll
    for (int s = 0; s < CS; ++s)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        cv[s][h] = buf_load16(csrc, static_cast<uint32_t>(s * 2048 + h * 1024 + lane * 16));
  } else {
    const auto xsrc = row_rsrc(x, static_cast<uint32_t>(K) * 2u);
#pragma unroll
    for (int s = 0; s < CS; ++s)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t off = static_cast<uint32_t>(s * 2048 + h * 1024 + lane * 16) * 2u;
        xv[s][h][0] = buf_load16(xsrc, off);
        xv[s][h][1] = buf_load16(xsrc, off + 16u);
      }
  }
  __builtin_amdgcn_sched_barrier(0);
  const int rows = min(R, N - row0);
  const auto wsrc = row_rsrc(qw + static_cast<int64_t>(row0) * K,
                             static_cast<uint32_t>(rows) * static_cast<uint32_t>(K));
  uint4 wv[R][CS][2];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int s = 0; s < CS; ++s)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        wv[r][s][h] = buf_load16_stream(
            wsrc, static_cast<uint32_t>(r * K + s * 2048 + h * 1024 + lane * 16));
  __builtin_amdgcn_sched_barrier(0);
  float scale;
  v8i bq[CS];
  if constexpr (CODES) {
    scale = sx[0];
#pragma unroll
    for (int s = 0; s < CS; ++s) bq[s] = to_v8i(cv[s][0], cv[s][1]);
  } else {
    uint32_t mm = 0;
#pragma unroll
    for (int s = 0; s < CS; ++s)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          mm = pk_max_u16(mm, bf16x2_abs_bits(xv[s][h][j].x));
          mm = pk_max_u16(mm, bf16x2_abs_bits(xv[s][h][j].y));
          mm = pk_max_u16(mm, bf16x2_abs_bits(xv[s][h][j].z));
          mm = pk_max_u16(mm, bf16x2_abs_bits(xv[s][h][j].w));
        }
    scale = row_scale(
        __uint_as_float(wave_max_u32(max(mm & 0xffffu, mm >> 16)) << 16));
    const RowDivisor d = make_divisor(scale);
#pragma unroll
    for (int s = 0; s < CS; ++s) {
      uint4 half[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint2 lo = quantize8(xv[s][h][0], d), hi = quantize8(xv[s][h][1], d);
        half[h] = make_uint4(lo.x, lo.y, hi.x, hi.y);
      }
      bq[s] = to_v8i(half[0], half[1]);
    }
  }
  m1_rows_mfma<CS, R>(wv, bq, scale, sw, N, row0, y);
}

template <int CS, int R, bool CODES>
__global__ __launch_bounds__(256) void gemv_m1_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ qx,
    const float* __restrict__ sx, const uint8_t* __restrict__ qw,
    const float* __restrict__ sw, int N, int K, uint16_t* __restrict__ y) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row0 = (static_cast<int>(blockIdx.x) * 4 + wave) * R;
  if (row0 >= N) return;
  m1_rows<CS, R, CODES>(x, qx, sx, qw, sw, N, K, y, row0);
}

// One token, K above what a wave can hold as a whole bf16 row in registers
// (K > 4096), for the grouped kernel: the workgroup's 4 waves share the
// row through LDS.  Every thread loads CS 16-byte chunks of x (chunk c =
// thread + 256 j), the waves' maxima meet in LDS, every thread quantizes its
// chunks with the quantizer's device functions into the LDS code row, and
// every wave then reads the codes of the whole row in the K-class layout and
// runs m1_rows_mfma: the same codes, scale and MFMA order as m1_rows, so the
// same bits.  Waves without rows (past N) still take part in the staging.
// LDS use: CS * 2048 code bytes + 16 (K <= 12288 in the grouped kernel).
constexpr int kGroupMaxSteps = 6;     // K <= 12288
constexpr int kGroupLdsBytes = kGroupMaxSteps * 2048 + 16;

template <int CS, int R>
__device__ __forceinline__ void m1_rows_lds(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ qw,
    const float* __restrict__ sw, int N, int K, uint16_t* __restrict__ y,
    int row0, uint8_t* __restrict__ codes, uint32_t* __restrict__ wmax) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tid = threadIdx.x;
  // The workgroup may have staged another row in the same LDS just before
  // (persistent grid): every wave is done reading it once all are here.
  lds_barrier();
  const auto xsrc = row_rsrc(x, static_cast<uint32_t>(K) * 2u);
  uint4 xv[CS];
#pragma unroll
  for (int j = 0; j < CS; ++j)
    xv[j] = buf_load16(xsrc, static_cast<uint32_t>(tid + 256 * j) * 16u);
  __builtin_amdgcn_sched_barrier(0);
  const int rows = max(0, min(R, N - row0));
  const auto wsrc = row_rsrc(qw + static_cast<int64_t>(min(row0, N)) * K,
                             static_cast<uint32_t>(rows) * static_cast<uint32_t>(K));
  uint4 wv[R][CS][2];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int s = 0; s < CS; ++s)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        wv[r][s][h] = buf_load16_stream(
            wsrc, static_cast<uint32_t>(r * K + s * 2048 + h * 1024 + lane * 16));
  __builtin_amdgcn_sched_barrier(0);
  uint32_t mm = 0;
#pragma unroll
  for (int j = 0; j < CS; ++j) {
    mm = pk_max_u16(mm, bf16x2_abs_bits(xv[j].x));
    mm = pk_max_u16(mm, bf16x2_abs_bits(xv[j].y));
    mm = pk_max_u16(mm, bf16x2_abs_bits(xv[j].z));
    mm = pk_max_u16(mm, bf16x2_abs_bits(xv[j].w));
  }
  const uint32_t wm = wave_max_u32(max(mm & 0xffffu, mm >> 16));
  if (lane == 0) wmax[wave] = wm;
  lds_barrier();
  const uint32_t am = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
  const float scale = row_scale(__uint_as_float(am << 16));
  const RowDivisor d = make_divisor(scale);
#pragma unroll
  for (int j = 0; j < CS; ++j)
    *reinterpret_cast<uint2*>(codes + (tid + 256 * j) * 8) = quantize8(xv[j], d);
  lds_barrier();
  if (rows <= 0) return;
  // Step-major, so that one step's codes are live at a time; each row's
  // accumulator still takes the steps in order (the bits of m1_rows_mfma).
  v4f acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int s = 0; s < CS; ++s) {
    const v8i bq = to_v8i(*reinterpret_cast<const uint4*>(codes + s * 2048 + lane * 16),
                          *reinterpret_cast<const uint4*>(codes + s * 2048 + 1024 + lane * 16));
#pragma unroll
    for (int r = 0; r < R; ++r)
      acc[r] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
          to_v8i(wv[r][s][0], wv[r][s][1]), bq, acc[r], 0, 0, 0, 0, 0, 0);
  }
  const int qd = (lane & 15) - 4 * (lane >> 4);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float dg = qd == 0 ? acc[r][0] : qd == 1 ? acc[r][1] : qd == 2 ? acc[r][2]
             : qd == 3 ? acc[r][3] : 0.0f;
    dg = wave_sum_to_63(dg);
    const int n = row0 + r;
    if (lane == 63 && n < N) y[n] = f32_to_bf16_bits(dg * sw[n] * scale);
  }
}

// Grouped one-token Linears: up to kGroupMax independent FP8_DYNAMIC
// Linears at M = 1, K <= 12288, in one launch (a whole decode layer's weight stream with
// one ramp-up and one tail instead of one per Linear).  The grid is the
// concatenation of the items' work units, each item a contiguous run of
// units of 4 waves, R rows per wave; items with K <= 4096 run m1_rows
// (barrier-free), longer ones m1_rows_lds.  Every item's output equals,
// bit for bit, what gemv_m1_kernel gives for it alone.
struct GroupItem {
  const uint16_t* x;
  const uint8_t* qw;
  const float* sw;
  uint16_t* y;
  int n, k;
  int wg0;    // first workgroup of the item
  int rpw;    // rows per wave
};
struct GroupArgs {
  GroupItem it[kGroupMax];
  int count;
  int units;  // workgroup-sized work units over all items
};

template <int CS, int R>
__device__ __forceinline__ void group_item(const GroupItem& g, int row0,
                                           uint8_t* codes, uint32_t* wmax) {
  if constexpr (CS <= 2) {
    if (row0 < g.n)
      m1_rows<CS, R, false>(g.x, nullptr, nullptr, g.qw, g.sw, g.n, g.k, g.y, row0);
  } else {
    m1_rows_lds<CS, R>(g.x, g.qw, g.sw, g.n, g.k, g.y, row0, codes, wmax);
  }
}

// Rows per wave in the grouped kernel: four for the register-held rows
// (K <= 4096), one for the rows staged through LDS.  Measured on the decode
// layer in one launch (7 Linears, 193 MB): the 6 K = 4096 Linears take
// 27.9 us with four rows per wave against 31.2 with two (the one-Linear
// launches prefer two: a grouped launch has work enough to fill the GPU
// with fewer, longer waves).  Two rows per wave for down would take it
// from 12.8 to 11.3 us alone, but its registers lower the whole kernel's
// occupancy and the layer then takes 38.3 us against 34.9.  With the
// kernel held to 128 VGPRs (4 waves per SIMD, no spills) the layer takes
// 34.1 us.
constexpr int kGroupRowsRegs = 4;
constexpr int kGroupRowsLds = 1;

template <int CS>
__device__ __forceinline__ void group_cs(const GroupItem& g, int local_wg, int wave,
                                         uint8_t* codes, uint32_t* wmax) {
  constexpr int R = CS <= 2 ? kGroupRowsRegs : kGroupRowsLds;
  group_item<CS, R>(g, (local_wg * 4 + wave) * R, codes, wmax);
}

// A workgroup takes work units blockIdx.x, blockIdx.x + gridDim.x, ...
// (a persistent grid of at most a few workgroups per CU: dispatching
// thousands of short workgroups costs more than looping).
__global__ __launch_bounds__(256, 4) void gemv_group_kernel(const GroupArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t codes[kGroupLdsBytes];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint32_t* wmax = reinterpret_cast<uint32_t*>(codes + kGroupMaxSteps * 2048);
  for (int unit = static_cast<int>(blockIdx.x); unit < a.units;
       unit += static_cast<int>(gridDim.x)) {
    int i = 0;
    for (int j = 1; j < a.count; ++j)
      if (unit >= a.it[j].wg0) i = j;
    const GroupItem& g = a.it[i];
    const int local = unit - g.wg0;
    switch ((g.k + 2047) / 2048) {
      case 1: group_cs<1>(g, local, wave, codes, wmax); break;
      case 2: group_cs<2>(g, local, wave, codes, wmax); break;
      case 3: group_cs<3>(g, local, wave, codes, wmax); break;
      case 4: group_cs<4>(g, local, wave, codes, wmax); break;
      case 5: group_cs<5>(g, local, wave, codes, wmax); break;
      default: group_cs<6>(g, local, wave, codes, wmax); break;
    }
  }
}

// Rows per wave for gemv_m1_kernel.  Every wave reads the whole activation
// row (2 K bytes, from L2), so more rows per wave amortize it, fewer give
// more waves: measured on MI355X at K = 4096, one row per wave up to
// N = 2048 (k/v, 1024 x 4096: 3.0 us, against 4.9 us for the LDS-staged
// kernel) and two above (q 5.0 against 5.9 us, gate 10.6 against 12.1,
// packed qkv 6.4 against 7.4, packed gate_up 18.6 against 21.7); four or
// more rows per wave were 2-20 % slower.  With the test hooks on,
// FP8W8A8_GEMV_M1_ROWS overrides (a tuning aid; at most 8 items of 2 KB per
// wave).
int m1_rows_per_wave(int64_t n, int cs) {
  if (const char* e = test_hook("FP8W8A8_GEMV_M1_ROWS")) {
    const int v = std::atoi(e);
    if ((v == 1 || v == 2 || v == 4 || v == 8) && cs * v <= 8) return v;
  }
  return (n <= 2048 || cs * 2 > 8) ? 1 : 2;
}

struct M1Args {
  const uint16_t* x;
  const uint8_t* qx;
  const float* sx;
  const uint8_t* qw;
  const float* sw;
  int64_t n, k;
  uint16_t* y;
};

template <int CS, int R, bool CODES>
hipError_t launch_m1(const M1Args& a, hipStream_t stream) {
  const int64_t waves = (a.n + R - 1) / R;
  gemv_m1_kernel<CS, R, CODES><<<dim3(static_cast<uint32_t>((waves + 3) / 4)), dim3(256),
                                 0, stream>>>(a.x, a.qx, a.sx, a.qw, a.sw,
                                              static_cast<int>(a.n),
                                              static_cast<int>(a.k), a.y);
  return hipGetLastError();
}

template <int CS, bool CODES>
hipError_t launch_m1_cs(const M1Args& a, hipStream_t stream) {
  switch (m1_rows_per_wave(a.n, CS)) {
    case 8: if constexpr (CS * 8 <= 8) return launch_m1<CS, 8, CODES>(a, stream); break;
    case 4: if constexpr (CS * 4 <= 8) return launch_m1<CS, 4, CODES>(a, stream); break;
    case 2: if constexpr (CS * 2 <= 8) return launch_m1<CS, 2, CODES>(a, stream); break;
    default: break;
  }
  return launch_m1<CS, 1, CODES>(a, stream);
}

}  // namespace detail

// The barrier-free M = 1 kernel runs by default for K <= 4096 (two steps):
// at K = 12288 (down) the activation row each wave re-reads is twice its
// weight bytes, and it measured 14.4 us against 11.7 us for the LDS-staged
// kernel.  With the test hooks on, FP8W8A8_GEMV_M1=0 switches it off, =1
// takes it up to K = 16384 (comparison and test aids; where the LDS-staged kernel gives waves whole
// rows the two give the same bits).
bool gemv_m1_fits(int64_t m, int64_t k) {
  if (m != 1 || k > 8 * 2048) return false;
  const char* e = test_hook("FP8W8A8_GEMV_M1");
  if (e && e[0] == '0') return false;
  if (e && e[0] == '1') return true;
  return k <= 2 * 2048;
}

template <bool CODES>
hipError_t launch_gemv_m1(const M1Args& a, hipStream_t stream) {
  switch ((a.k + 2047) / 2048) {
    case 1: return launch_m1_cs<1, CODES>(a, stream);
    case 2: return launch_m1_cs<2, CODES>(a, stream);
    case 3: return launch_m1_cs<3, CODES>(a, stream);
    case 4: return launch_m1_cs<4, CODES>(a, stream);
    case 5: return launch_m1_cs<5, CODES>(a, stream);
    case 6: return launch_m1_cs<6, CODES>(a, stream);
    case 7: return launch_m1_cs<7, CODES>(a, stream);
    case 8: return launch_m1_cs<8, CODES>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemv(const uint16_t* x, int64_t ldx, const uint8_t* qx,
                       const float* sx, const uint8_t* qw, const float* sw,
                       int64_t m, int64_t n, int64_t k, uint16_t* y,
                       int64_t ldy, hipStream_t stream) {
  if (m == 0 || n == 0) return hipSuccess;
  const GemvPlan pl = plan_gemv(m, n, k);
  const GemvPre none{nullptr, 0, 0.0f};
  if (x != nullptr) {
    if (!gemv_fused_fits(m, n, k)) return hipErrorInvalidValue;
    if (gemv_m1_fits(m, k))
      return launch_gemv_m1<false>(M1Args{x, nullptr, nullptr, qw, sw, n, k, y}, stream);
    return launch_one<2, kFusedRegs>(x, ldx, qx, sx, qw, sw, m, pl.lg_mp, n, k,
                                     pl.gpw, pl.ni, y, ldy, none, stream);
  }
  if (gemv_m1_fits(m, k))
    return launch_gemv_m1<true>(M1Args{nullptr, qx, sx, qw, sw, n, k, y}, stream);
  if (m * ((k + 1023) / 1024 * 1024 + kLdsRowPad) <= kStageLds)
    return launch_one<1, 1>(x, ldx, qx, sx, qw, sw, m, pl.lg_mp, n, k, pl.gpw,
                            pl.ni, y, ldy, none, stream);
  return launch_one<0, 1>(x, ldx, qx, sx, qw, sw, m, pl.lg_mp, n, k, pl.gpw,
                          pl.ni, y, ldy, none, stream);
}

// Whether the pre-step runs inside the LDS-staged GEMV's activation
// staging.  Not at one token where the barrier-free M = 1 kernel takes the
// shape: there the stand-alone pre-step kernel followed by that kernel on
// the codes is faster (measured per decode layer with both fusions: 47.4 us
// against 48.2 us with the norm in the staging), and gives the same bits.
hipError_t launch_gemv_group_m1(const GroupLinear* items, int count,
                                hipStream_t stream) {
  if (count < 1 || count > kGroupMax) return hipErrorInvalidValue;
  GroupArgs a{};
  a.count = count;
  int64_t wgs = 0;
  int order[kGroupMax];
  for (int i = 0; i < count; ++i) order[i] = i;
  if (const char* e = test_hook("FP8W8A8_GROUP_SORT")) {
    if (e[0] == '1')  // longest rows first
      std::stable_sort(order, order + count, [&](int p, int q) {
        return items[p].k > items[q].k;
      });
  }
  for (int i = 0; i < count; ++i) {
    const GroupLinear& L = items[order[i]];
    const int cs = static_cast<int>((L.k + 2047) / 2048);
    if (cs > kGroupMaxSteps) return hipErrorInvalidValue;
    const int rpw = cs <= 2 ? kGroupRowsRegs : kGroupRowsLds;
    a.it[i] = GroupItem{L.x, L.qw, L.sw, L.y, static_cast<int>(L.n),
                        static_cast<int>(L.k), static_cast<int>(wgs), rpw};
    wgs += (L.n + 4 * rpw - 1) / (4 * rpw);
  }
  if (wgs <= 0 || wgs > (int64_t{1} << 31) - 1) return hipErrorInvalidValue;
  a.units = static_cast<int>(wgs);
  int64_t grid = wgs;
  if (const char* e = test_hook("FP8W8A8_GROUP_GRID")) {
    const int64_t v = std::atoll(e);
    if (v >= 1) grid = std::min(grid, v);
  }
  gemv_group_kernel<<<dim3(static_cast<uint32_t>(grid)), dim3(256), 0, stream>>>(a);
  return hipGetLastError();
}

bool gemv_pre_fits(int pre, int64_t m, int64_t n, int64_t k) {
  if (!gemv_fused_fits(m, n, k) || m > kGemvMaxM) return false;
  if (gemv_m1_fits(m, k)) return false;
  if (pre == kPreRmsNorm) return k % 512 == 0 && k / 512 <= kMaxNormBlocksPerRow;
  return pre == kPreSwiGlu;
}

hipError_t launch_gemv_pre(int pre, const uint16_t* x, int64_t ldx,
                           const uint16_t* x2, int64_t ld2, float eps,
                           const uint8_t* qw, const float* sw, int64_t m,
                           int64_t n, int64_t k, uint16_t* y, int64_t ldy,
                           hipStream_t stream) {
  if (m == 0 || n == 0) return hipSuccess;
  if (!gemv_pre_fits(pre, m, n, k)) return hipErrorInvalidValue;
  const GemvPlan pl = plan_gemv(m, n, k);
  const GemvPre extra{x2, ld2, eps};
  if (pre == kPreRmsNorm)
    return launch_one<3, kFusedRegs>(x, ldx, nullptr, nullptr, qw, sw, m, pl.lg_mp,
                                     n, k, pl.gpw, pl.ni, y, ldy, extra, stream);
  return launch_one<4, kFusedRegs>(x, ldx, nullptr, nullptr, qw, sw, m, pl.lg_mp, n,
                                   k, pl.gpw, pl.ni, y, ldy, extra, stream);
}

}  // namespace fp8w8a8
