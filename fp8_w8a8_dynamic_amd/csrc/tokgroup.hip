// Grouped FP8_DYNAMIC Linears on given codes for a few tokens (1 <= M <= 256),
// up to kGroupMax of them in one persistent launch: per-token E4M3 codes and
// scales times channel-wise E4M3 weights, float32 accumulation, bf16 output
// through the token-scale x channel-scale epilogue (MOSS-VL quantization
// README, "FP8-Dynamic").  At these token counts every Linear is bound by
// its weight bytes (MOSS-VL-Realtime-FP8 article, on why the model is
// quantized), and a run of small launches pays a ramp-up and a tail per
// launch; Linears that read the same activations can share one code buffer
// and go out as one stream.
//
// Weights in MFMA tiles.  Offline, next to the quantization, a Linear's
// [N, K] codes are permuted (tile_weights_kernel) so that each MFMA item --
// 16 weight rows x 128 K bytes -- is one contiguous 2 KB tile laid out in
// the order the lanes take it: tile byte h * 1024 + 16 l + e holds row
// 16 rb + (l & 15), K byte 128 i + 64 h + 16 (l >> 4) + e of item i of row
// block rb.  The tiles are grouped in K panels of four items (512 bytes of
// K, the stage of the kernel below up to 64 tokens): panel p holds the
// tiles of every row block for its K range, row block by row block, and
// the panels follow each other in K order.  A wave then fetches an item
// with two fully contiguous 1 KB loads, four items (a stage) are 8 KB of
// consecutive memory, and the stages that all workgroups of a launch
// stream at one time lie side by side in one panel instead of one row
// block's length apart.  (Row-major rows fetched 64 bytes at a time from 16
// rows per load instruction measured ~25 % slower for the same bytes; with
// the tiles of each row block contiguous over the whole K, 8 KB stages
// 64 KB apart, the bare weight stream of a 512-workgroup launch at 8
// stages per wave ran at 5.6 TB/s against 6.05 in panel order.)
//
// Work decomposition.  A work unit is 64 consecutive weight rows (four row
// blocks) of one item over the item's whole K; each of the four waves of a
// workgroup owns one row block.  K is walked in stages of 512 bytes (four
// MFMA items).  A stage's weights are requested into registers D stages
// ahead (a ring of D + 1 slots, or of D slots refilled item by item as
// the MFMAs take them); its codes (16 T token rows x 512 bytes,
// T = ceil(M / 16), each thread a 16-byte share) one or two stages ahead,
// into registers, and written to LDS one step before their use, where the
// four waves read them.  A weight fragment feeds T MFMAs, one per block of 16
// tokens, so the codes cross L2 once per 64 weight rows.  A workgroup walks
// its units as one stream of stages: the next unit's first stages are in
// flight while the current unit finishes.  Units are numbered longest K
// first and dealt out in rounds of gridDim.x.  Workgroups start in index
// order, so among equal units the low indices finish first; round r + 1
// starts at the first workgroup that held a unit of round 0's shortest
// length (a shift of that many workgroups per round; 0 when all units
// are equal).  In a decoder layer at a few tokens, down's 64 units at
// K = 12288 (24 stages) go to workgroups 0-63 and the units past the
// first round to workgroups 64, 65, ..., which hold 8-stage units.  No
// workgroup waits on another and no partial sums leave the wave: each
// output is one lane's accumulator, items in K order.
//
// MFMA layout (v_mfma_f32_16x16x128_f8f6f4): lane (r, g) = (l & 15, l >> 4)
// holds, of each 128-byte item, bytes 16 g .. 16 g + 15 and 64 + 16 g .. +15
// of weight row r (A) and of token r of the block (B), the same K order on
// both operands; accumulator entry q of lane l is (weight row 4 g + q, token
// r).  LDS rows are 512 bytes per token with the 16-byte chunks XOR-swizzled
// by the token's low four bits, so the 16 lanes of one chunk column read 16
// distinct bank groups.
//
// Out-of-range bytes read as 0 through buffer descriptors: tokens past M
// (the codes' descriptor covers M * K bytes), the K tail of a last stage
// (offsets moved past the descriptor), outputs of tokens past M (dropped by
// the output's descriptor, M * N values).  A unit's outputs leave through
// LDS as whole 128-byte row segments.
#include <algorithm>
#include <cstdlib>
#include <utility>

#include "device_common.h"
#include "launch.h"

namespace fp8w8a8 {

namespace tokgroup {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr uint32_t kPastEnd = 0x80000000u;  // an offset past every descriptor
constexpr int kDepth = 2;                   // stages of weights requested ahead (T <= 4)

// Stage geometry per token-block count T (16 T token rows): a stage is IPS
// MFMA items of 128 K bytes, so that two stages of codes (16 T x 128 IPS
// bytes each) fit LDS: 4 items up to 64 tokens, 2 up to 128, 1 up to 256.
constexpr int ips_of(int T) { return T <= 4 ? 4 : (T <= 8 ? 2 : 1); }
constexpr int sb_of(int T) { return 128 * ips_of(T); }    // stage bytes
constexpr int nx_of(int T) { return T * ips_of(T) / 2; }  // 16-byte code slots per thread
// Weights requested this many stages ahead: 16 KB per wave in flight at
// T <= 8, 14 KB at T = 16.
constexpr int depth_of(int T) { return T <= 4 ? kDepth : (T <= 8 ? 4 : 7); }
// Chunk swizzle of a token's LDS row: rows of 32 or 16 chunks take the
// token's low four bits; rows of 8 chunks (128 bytes, two rows per 256-byte
// bank line) take bits 1-3, so that the 16 tokens of a block read the same
// logical chunk from 16 distinct bank groups either way.
template <int T>
__device__ __forceinline__ int code_swz(int tok) {
  return ips_of(T) >= 2 ? (tok & 15) : ((tok >> 1) & 7);
}

struct Item {
  const uint8_t* qx;  // codes of the item's first K byte (row stride ldx)
  const float* sx;
  const uint8_t* qw;  // tiled (panel order) codes of the whole Linear: n / 16 x kbt tiles
  const float* sw;
  uint16_t* y;
  float* part;  // non-null: raw float32 sums [M, n] here instead of y
  int n, k;     // k: the K range the item sums over
  int ldx;      // bytes between token rows of the codes (>= k)
  int kb0;      // the item's first K block (128 bytes) in the tiled Linear
  int kbt;      // K blocks of the tiled Linear (>= kb0 + k / 128)
  int u0;       // first work unit of the item
};
struct Args {
  Item it[kGroupMax];
  int count;
  int units;
  int m;
  int shift;  // workgroups by which each round's deal turns (0 <= shift < grid)
  int sb;     // stage bytes (sb_of(T))
};

__device__ __forceinline__ v8i to_v8i(uint4 lo, uint4 hi) {
  v8i r;
  r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
  r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
  return r;
}

__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Wave-uniform position in a workgroup's stream of stages.
struct Cursor {
  int unit, stage, item, stages;
};

__device__ __forceinline__ void cursor_at(Cursor& c, const Args& a, int unit) {
  c.unit = unit;
  c.stage = 0;
  c.item = 0;
  for (int j = 1; j < a.count; ++j)
    if (unit >= a.it[j].u0) c.item = j;
  c.stages = (a.it[c.item].k + a.sb - 1) / a.sb;
}

// The workgroup's unit after u: round r holds units r G .. r G + G - 1, and
// workgroup b takes unit r G + ((b - r shift) mod G) of it.
__device__ __forceinline__ int next_unit(int u, int shift) {
  const int G = static_cast<int>(gridDim.x), b = static_cast<int>(blockIdx.x);
  const int r = u / G + 1;
  return r * G + (b + G - (r % G) * shift % G) % G;
}

__device__ __forceinline__ void cursor_next(Cursor& c, const Args& a) {
  if (++c.stage == c.stages) cursor_at(c, a, next_unit(c.unit, a.shift));
}

// The epilogue's scales for a unit: sw of rows 4 g .. 4 g + 3 of the wave's
// row block, sx of token r of each token block.
template <int T>
struct Scales {
  float4 w;
  float x[T];
};

// A stage's weight fragments in one wave's registers.
template <int T>
struct Weights {
  uint4 w[ips_of(T)][2];
};
// This thread's share of a stage's codes (LDS slots j * 256 + tid).
template <int T>
struct Codes {
  uint4 x[nx_of(T)];
};

// Requests for stage c.  When `live` is false the same instructions go out
// with offsets past the descriptors' ends (nothing is read), so the
// instruction stream -- and with it every wait count -- is the same on
// every path.
template <int T>
__device__ __forceinline__ void load_codes(Codes<T>& xc, const Args& a, const Cursor& c,
                                           bool live, int M, int tid) {
  const Item& it = a.it[c.item];
  const int K = it.k;
  constexpr int CPR = sb_of(T) / 16;  // 16-byte chunks per token row
  const int k0 = c.stage * sb_of(T);
  // The descriptor ends with token M - 1's last byte of the K range, so
  // tokens past M read as zero.
  const auto xr = row_rsrc(it.qx, static_cast<uint32_t>((M - 1) * it.ldx + K));
#pragma unroll
  for (int j = 0; j < nx_of(T); ++j) {
    // LDS slot p (16 bytes) = token p / CPR, chunk (p % CPR) ^ swizzle.
    const int p = j * 256 + tid;
    const int tok = p / CPR;
    const int ch = (p % CPR) ^ code_swz<T>(tok);
    const bool ok = live && k0 + (ch >> 3) * 128 < K && tok < M;
    xc.x[j] = buf_load16(xr, ok ? static_cast<uint32_t>(tok * it.ldx + k0 + ch * 16)
                                : kPastEnd);
  }
}

// Item i of stage c's weights for this wave: its 2 KB tile in the panel
// order (panel p = ib / 4 holds ipp tiles of every row block, row block by
// row block; all wave-uniform).
template <int T>
__device__ __forceinline__ void load_weight_item(uint4 (&w)[2], const Args& a, const Cursor& c,
                                                 bool live, int i, int wave, int lane) {
  const Item& it = a.it[c.item];
  const int k0 = c.stage * sb_of(T);
  // The wave's row block; its 2 KB tiles lie one per K block, in the K panels.
  const int rb = (c.unit - it.u0) * 4 + wave;
  const bool ok = live && k0 + i * 128 < it.k;
  const int ib = it.kb0 + (ok ? k0 / 128 + i : 0);
  const int p = ib >> 2, ipp = min(4, it.kbt - 4 * p);
  const auto wr = row_rsrc(it.qw + static_cast<int64_t>(p) * it.n * 512 +
                               (static_cast<int64_t>(rb) * ipp + (ib & 3)) * 2048,
                           2048u);
#pragma unroll
  for (int h = 0; h < 2; ++h)
    w[h] = buf_load16_stream(wr, ok ? static_cast<uint32_t>(h * 1024 + lane * 16) : kPastEnd);
}

// A whole stage (the same addresses as load_weight_item for each item;
// written out here, as routing it through the per-item helper made the
// compiler keep the T = 8 ring in scratch).
template <int T>
__device__ __forceinline__ void load_weights(Weights<T>& s, const Args& a, const Cursor& c,
                                             bool live, int wave, int lane) {
  const Item& it = a.it[c.item];
  const int K = it.k;
  const int k0 = c.stage * sb_of(T);
  const int rb = (c.unit - it.u0) * 4 + wave;
#pragma unroll
  for (int i = 0; i < ips_of(T); ++i) {
    const bool ok = live && k0 + i * 128 < K;
    const int ib = it.kb0 + (ok ? k0 / 128 + i : 0);
    const int p = ib >> 2, ipp = min(4, it.kbt - 4 * p);
    const auto wr = row_rsrc(it.qw + static_cast<int64_t>(p) * it.n * 512 +
                                 (static_cast<int64_t>(rb) * ipp + (ib & 3)) * 2048,
                             2048u);
#pragma unroll
    for (int h = 0; h < 2; ++h)
      s.w[i][h] = buf_load16_stream(wr, ok ? static_cast<uint32_t>(h * 1024 + lane * 16)
                                           : kPastEnd);
  }
}

template <int T>
__device__ __forceinline__ void load_scales(Scales<T>& sc, const Args& a, const Cursor& c,
                                            int M, int wave, int lane) {
  const Item& it = a.it[c.item];
  const int r = lane & 15, g = lane >> 4;
  sc.w = *reinterpret_cast<const float4*>(it.sw + (c.unit - it.u0) * 64 + wave * 16 + 4 * g);
#pragma unroll
  for (int t = 0; t < T; ++t) sc.x[t] = it.sx[min(16 * t + r, M - 1)];
}

template <int T>
__device__ __forceinline__ void store_codes(const Codes<T>& xc, uint8_t* xs, int tid) {
#pragma unroll
  for (int j = 0; j < nx_of(T); ++j)
    *reinterpret_cast<uint4*>(xs + (j * 256 + tid) * 16) = xc.x[j];
}

template <int T>
__device__ __forceinline__ void compute_stage(v4f (&acc)[T], const Weights<T>& s,
                                              const uint8_t* xs, int lane) {
  const int r = lane & 15, g = lane >> 4;
  // (Token 16 t + r has the swizzle of r: blocks start at multiples of 16.)
  const int sw = code_swz<T>(r);
  // Token fragment of MFMA j of the stage (item j / T, token block j % T).
  auto frag = [&](int j) {
    const int i = j / T, t = j % T;
    const uint8_t* row = xs + (16 * t + r) * sb_of(T);
    const uint4 lo = *reinterpret_cast<const uint4*>(row + (((i * 8 + g) ^ sw) * 16));
    const uint4 hi = *reinterpret_cast<const uint4*>(row + (((i * 8 + 4 + g) ^ sw) * 16));
    return to_v8i(lo, hi);
  };
  if constexpr (T <= 4) {
#pragma unroll
    for (int i = 0; i < ips_of(T); ++i) {
      const v8i a = to_v8i(s.w[i][0], s.w[i][1]);
#pragma unroll
      for (int t = 0; t < T; ++t)
        acc[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            a, frag(i * T + t), acc[t], 0, 0, 0, 0, 0, 0);
      // One item's fragments at a time (hoisting every LDS read of the
      // stage would hold 4 x 8 T registers).
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    // Many token blocks per item: the fragments are read kAhead MFMAs
    // ahead through a small ring, the order pinned (left to itself the
    // compiler read each fragment right before its MFMA and waited for it,
    // one LDS round trip per MFMA).
    constexpr int kN = ips_of(T) * T, kAhead = 4;
    v8i ring[kAhead + 1];
#pragma unroll
    for (int j = 0; j < kAhead; ++j) ring[j] = frag(j);
#pragma unroll
    for (int j = 0; j < kN; ++j) {
      if (j + kAhead < kN) ring[(j + kAhead) % (kAhead + 1)] = frag(j + kAhead);
      const int i = j / T, t = j % T;
      acc[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
          to_v8i(s.w[i][0], s.w[i][1]), ring[j % (kAhead + 1)], acc[t], 0, 0, 0, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// compute_stage with a rolling refill (T <= 4): right after item i's MFMAs
// have taken its weight fragment, item i of stage c (the stage D slots
// later) is requested into the same registers, so D stage slots keep D
// stages of weights in flight where the requests at the top of a step
// need D + 1 (same MFMAs in the same order: the same bits).
template <int T>
__device__ __forceinline__ void compute_stage_refill(v4f (&acc)[T], Weights<T>& s,
                                                     const uint8_t* xs, int lane,
                                                     const Args& a, const Cursor& c,
                                                     bool live, int wave) {
  static_assert(T <= 4, "one item's fragments at a time");
  const int r = lane & 15, g = lane >> 4;
  const int sw = code_swz<T>(r);
  auto frag = [&](int j) {
    const int i = j / T, t = j % T;
    const uint8_t* row = xs + (16 * t + r) * sb_of(T);
    const uint4 lo = *reinterpret_cast<const uint4*>(row + (((i * 8 + g) ^ sw) * 16));
    const uint4 hi = *reinterpret_cast<const uint4*>(row + (((i * 8 + 4 + g) ^ sw) * 16));
    return to_v8i(lo, hi);
  };
#pragma unroll
  for (int i = 0; i < ips_of(T); ++i) {
    const v8i wa = to_v8i(s.w[i][0], s.w[i][1]);
#pragma unroll
    for (int t = 0; t < T; ++t)
      acc[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
          wa, frag(i * T + t), acc[t], 0, 0, 0, 0, 0, 0);
    load_weight_item<T>(s.w[i], a, c, live, i, wave, lane);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// One token's 64 outputs of a unit in LDS (bf16), padded so that the 16
// tokens of a write land in 16 distinct bank groups.
constexpr int kOutRow = 64 * 2 + 16;

// The unit's 16 T x 64 outputs: scaled, rounded to bf16 and staged in LDS by
// the four waves (token 16 t + r, channels 16 wave + 4 g .. + 3 per lane),
// then written out as whole 128-byte row segments, 16 bytes per thread
// (tokens past M dropped by the output's descriptor).  Every wave is at its
// unit's last stage here, so the barrier is met by all four; the next write
// to `ob` is a later unit's, after at least one more step's barrier.
template <int T>
__device__ __forceinline__ void epilogue(v4f (&acc)[T], const Scales<T>& sc,
                                         const Args& a, const Cursor& c, int M,
                                         int wave, int tid, uint8_t* ob) {
  const Item& it = a.it[c.item];
  const int N = it.n;
  const int lane = tid & 63, r = lane & 15, g = lane >> 4;
  if (it.part != nullptr) {
    // A K range of a split Linear: the raw sums, 4 consecutive channels of
    // a token per lane (tokens past M dropped by the descriptor).  The
    // branch is uniform over the workgroup and takes no barrier.
    const int n0 = (c.unit - it.u0) * 64 + 16 * wave + 4 * g;
    const auto pr = row_rsrc(it.part, static_cast<uint32_t>(M * N) * 4u);
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const v4f v = acc[t];
      // Default cache policy: the reduction reads them back right away.
      __builtin_amdgcn_raw_buffer_store_b128(
          v4u32_t{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                  __float_as_uint(v[3])},
          pr, static_cast<int>(((16 * t + r) * N + n0) * 4), 0, 0);
      acc[t] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    }
    return;
  }
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const v4f v = acc[t];
    const float xs = sc.x[t];
    uint2 pk;
    pk.x = pack_bf16x2(v[0] * sc.w.x * xs, v[1] * sc.w.y * xs);
    pk.y = pack_bf16x2(v[2] * sc.w.z * xs, v[3] * sc.w.w * xs);
    *reinterpret_cast<uint2*>(ob + (16 * t + r) * kOutRow + (16 * wave + 4 * g) * 2) = pk;
    acc[t] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  }
  lds_barrier();
  const int n0 = (c.unit - it.u0) * 64;
  const auto yr = row_rsrc(it.y, static_cast<uint32_t>(M * N) * 2u);
#pragma unroll
  for (int j = 0; j < (T + 1) / 2; ++j) {
    const int p = j * 256 + tid;
    const int tok = p >> 3, ch = p & 7;
    if (tok < 16 * T) {
      const uint4 v = *reinterpret_cast<const uint4*>(ob + tok * kOutRow + ch * 16);
      buf_store16(v, yr, static_cast<uint32_t>((tok * N + n0 + ch * 8) * 2));
    }
  }
}

// Step I of the stream (I counts modulo lcm(D + 1, 2)), computing stage C,
// with the codes requested DC stages ahead (ring slot (stage) % DC of X).
// Vector-memory requests complete in order, so the issue order carries the
// pipeline: the codes of stage C + DC go out first, then the weights of
// stage C + D (ring slot (I + D) % (D + 1)).  Stage C is computed from
// weight slot I % (D + 1) and LDS buffer I % 2; then the codes of C + 1 are
// written to LDS buffer (I + 1) % 2 (nobody reads it since the previous
// step's barrier) -- the wait for them also completes the weights
// requested before them and leaves the later requests in flight.  Every
// request is one the compiler tracks, so the waits it places are exact.
// Returns false once C was the workgroup's last stage.
// Weight stage slots: D + 1 when a step requests its stage at the top, D
// with the rolling refill (RR).
constexpr int slots_of(int D, bool RR) { return RR ? D : D + 1; }

template <int I, int T, int D, int DC, bool RR>
__device__ __forceinline__ bool step(v4f (&acc)[T], Weights<T> (&S)[slots_of(D, RR)],
                                     Codes<T> (&X)[DC], uint8_t (*xs)[16 * T * sb_of(T)],
                                     uint8_t* ob, Cursor (&Q)[D + 1], const Args& a, int M,
                                     int wave, int tid) {
  static_assert(DC >= 1 && DC <= D, "codes at most as far ahead as the weights");
  constexpr int NS = slots_of(D, RR);
  // Q[0] = C, Q[j] = C + j (a unit past the end once the units run out).
  const int lane = tid & 63;
  const bool more1 = Q[1].unit < a.units, moreC = Q[DC].unit < a.units,
             moreD = Q[D].unit < a.units;
  const bool last = Q[0].stage == Q[0].stages - 1;
  // The epilogue's scales first: waiting for them completes nothing issued
  // after them.
  Scales<T> sc;
  if (last) load_scales(sc, a, Q[0], M, wave, lane);
  load_codes(X[I % DC], a, moreC ? Q[DC] : Q[0], moreC, M, tid);
  if constexpr (!RR)
    load_weights(S[(I + D) % NS], a, moreD ? Q[D] : Q[0], moreD, wave, lane);
  // Keep the requests ahead of the MFMAs (the scheduler would otherwise
  // sink them below).
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (RR)
    compute_stage_refill(acc, S[I % NS], xs[I % 2], lane, a, moreD ? Q[D] : Q[0], moreD,
                         wave);
  else
    compute_stage(acc, S[I % NS], xs[I % 2], lane);
  if (last) epilogue(acc, sc, a, Q[0], M, wave, tid, ob);
  if (!more1) return false;
  store_codes(X[(I + 1) % DC], xs[(I + 1) % 2], tid);
  lds_barrier();
#pragma unroll
  for (int j = 0; j < D; ++j) Q[j] = Q[j + 1];
  if (moreD) cursor_next(Q[D], a);
  return true;
}

template <int T, int D, int DC, bool RR, int... Is>
__device__ __forceinline__ bool steps(std::integer_sequence<int, Is...>, v4f (&acc)[T],
                                      Weights<T> (&S)[slots_of(D, RR)], Codes<T> (&X)[DC],
                                      uint8_t (*xs)[16 * T * sb_of(T)], uint8_t* ob,
                                      Cursor (&Q)[D + 1], const Args& a, int M, int wave,
                                      int tid) {
  return (step<Is, T, D, DC, RR>(acc, S, X, xs, ob, Q, a, M, wave, tid) && ...);
}

// Vector-memory requests complete in order, so a step's closing wait for
// the codes of stage C + 1 also completes every weight request issued
// before them: at that point only DC stages of weights stay in flight.
// DC = 1: two workgroups per CU (two waves per SIMD, 256 registers each).
// DC = 2: the codes two stages ahead as well; at T <= 2 that still fits
// two workgroups per CU, at T = 3 or 4 it takes one (a wave's registers
// beyond 256) and is chosen for launches of at most one unit per CU.
// RR (T <= 4): the weights refilled item by item as each stage's MFMAs
// take them (compute_stage_refill), so D slots hold what D + 1 held; the
// registers freed take the second stage of codes, and DC = 2 fits two
// workgroups per CU at T = 3 and 4 too.
template <int T, int D, int DC, bool RR>
constexpr int tok_group_wg_per_cu() {
  return T <= 2 || ((DC == 1 || RR) && T <= 4) ? 2 : 1;
}
template <int T, int D, int DC, bool RR>
__global__ __launch_bounds__(256, (tok_group_wg_per_cu<T, D, DC, RR>())) void tok_group_kernel(
    const Args a) {
  static_assert(!RR || T <= 4, "the rolling refill reads one item's fragments at a time");
  __shared__ __attribute__((aligned(16))) uint8_t xs[2][16 * T * sb_of(T)];
  __shared__ __attribute__((aligned(16))) uint8_t ob[16 * T * kOutRow];
  const int tid = static_cast<int>(threadIdx.x);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int M = a.m;
  if (static_cast<int>(blockIdx.x) >= a.units) return;
  // Q[0]: the stage computed; Q[1..D]: the next D (a unit past the end once
  // the workgroup's units run out).
  Cursor Q[D + 1];
  cursor_at(Q[0], a, static_cast<int>(blockIdx.x));
#pragma unroll
  for (int j = 1; j <= D; ++j) {
    Q[j] = Q[j - 1];
    if (Q[j].unit < a.units) cursor_next(Q[j], a);
  }
  Weights<T> S[slots_of(D, RR)];
  Codes<T> X[DC];
  v4f acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  // Codes of stage 0 (into LDS buffer 0), weights of stages 0 .. D - 1 and
  // codes of stages 1 .. DC - 1 in flight.
  load_codes(X[0], a, Q[0], true, M, tid);
#pragma unroll
  for (int j = 0; j < D; ++j) {
    const bool live = Q[j].unit < a.units;
    load_weights(S[j], a, live ? Q[j] : Q[0], live, wave, lane);
  }
#pragma unroll
  for (int j = 1; j < DC; ++j) {
    const bool live = Q[j].unit < a.units;
    load_codes(X[j], a, live ? Q[j] : Q[0], live, M, tid);
  }
  store_codes(X[0], xs[0], tid);
  lds_barrier();
  constexpr int NS = slots_of(D, RR);
  constexpr int kPeriod = NS % 2 == 0 ? NS : 2 * NS;
  static_assert(kPeriod % DC == 0, "code ring period");
  while (steps<T, D, DC, RR>(std::make_integer_sequence<int, kPeriod>{}, acc, S, X, xs, ob,
                             Q, a, M, wave, tid)) {
  }
  // Nothing in flight when the workgroup leaves (the last requests read
  // nothing, but their registers go with the workgroup).
  __builtin_amdgcn_s_waitcnt(0);
}

template <int T, int D, int DC, bool RR = false>
hipError_t launch_d(Args a, hipStream_t stream) {
  // Two workgroups per CU where tok_group_wg_per_cu says so (LDS: 16 KB per
  // token block; registers: two waves per SIMD); otherwise one.  256 CUs.
  a.sb = sb_of(T);
  int64_t grid = std::min<int64_t>(a.units, tok_group_wg_per_cu<T, D, DC, RR>() * 256);
  if (const char* e = test_hook("FP8W8A8_TOKG_GRID")) {
    const int64_t v = std::atoll(e);
    if (v >= 1) grid = std::min<int64_t>(a.units, v);
  }
  // The deal's shift: how many of round 0's units (0 .. grid - 1, longest K
  // first) are longer than its last.
  const auto stages_of = [&](int unit) {
    int i = 0;
    for (int j = 1; j < a.count; ++j)
      if (unit >= a.it[j].u0) i = j;
    return (a.it[i].k + sb_of(T) - 1) / sb_of(T);
  };
  const int shortest = stages_of(static_cast<int>(grid) - 1);
  a.shift = 0;
  for (int i = 0; i < a.count && a.it[i].u0 < grid; ++i)
    if ((a.it[i].k + sb_of(T) - 1) / sb_of(T) > shortest) {
      const int end = i + 1 < a.count ? a.it[i + 1].u0 : a.units;
      a.shift += std::min<int>(end, static_cast<int>(grid)) - a.it[i].u0;
    }
  tok_group_kernel<T, D, DC, RR>
      <<<dim3(static_cast<uint32_t>(grid)), dim3(256), 0, stream>>>(a);
  return hipGetLastError();
}

// Codes two stages ahead at up to 32 tokens (two workgroups per CU either
// way); at 33-64 tokens the rolling refill (below), or with a test hook
// the earlier variants: codes two stages ahead when the launch has at most
// one unit per CU (then one workgroup per CU), else one stage ahead (two
// workgroups per CU); test hooks FP8W8A8_TOKG_CODES (1 or 2) and
// FP8W8A8_TOKG_DEPTH (2 or 3) override.
template <int T>
hipError_t launch_t(const Args& a, hipStream_t stream) {
  if constexpr (T == 3 || T == 4) {
    // 33-64 tokens: the rolling refill with the codes two stages ahead, two
    // workgroups per CU (the 36-layer stack at M = 64: 2.01 -> 1.93 ms per
    // pass).  Test hooks: FP8W8A8_TOKG_ROLL=0|1; with FP8W8A8_TOKG_CODES or
    // FP8W8A8_TOKG_DEPTH set (and no ROLL) the variants below run instead.
    const char* r = test_hook("FP8W8A8_TOKG_ROLL");
    const bool roll = r ? r[0] == '1'
                        : test_hook("FP8W8A8_TOKG_CODES") == nullptr &&
                              test_hook("FP8W8A8_TOKG_DEPTH") == nullptr;
    if (roll) return launch_d<T, kDepth, 2, true>(a, stream);
  }
  const char* c = test_hook("FP8W8A8_TOKG_CODES");
  const int dc = c ? std::atoi(c) : (T > 4 || T <= 2 || a.units <= 256 ? 2 : 1);
  if constexpr (T > 4) {
    if (dc == 1) return launch_d<T, depth_of(T), 1>(a, stream);
    if constexpr (T == 16)
      if (dc == 4) return launch_d<T, depth_of(T), 4>(a, stream);
    return launch_d<T, depth_of(T), 2>(a, stream);
  } else {
    const char* e = test_hook("FP8W8A8_TOKG_DEPTH");
    const int d = e ? std::atoi(e) : kDepth;
    if (dc == 2)
      return d == 3 ? launch_d<T, 3, 2>(a, stream) : launch_d<T, 2, 2>(a, stream);
    return d == 3 ? launch_d<T, 3, 1>(a, stream) : launch_d<T, 2, 1>(a, stream);
  }
}

// The MFMA-tile permutation of a row-major [n, k] code matrix: one thread
// per 16 bytes of the output.  K panel p (four 128-byte K blocks, fewer in
// the last) starts at byte p * n * 512 and holds, row block by row block,
// the panel's ipp tiles of each; tile byte h * 1024 + 16 l of tile (rb, i)
// takes row 16 rb + (l & 15), bytes 128 i + 64 h + 16 (l >> 4) .. + 15.
__global__ __launch_bounds__(256) void tile_weights_kernel(const uint8_t* __restrict__ qw,
                                                           int64_t chunks, int64_t n, int k,
                                                           uint8_t* __restrict__ out) {
  const int ki = k / 128;
  const int64_t panel_chunks = n * 32;  // n * 512 bytes
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t c = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; c < chunks;
       c += stride) {
    const int l = static_cast<int>(c & 63);
    const int h = static_cast<int>((c >> 6) & 1);
    const int p = static_cast<int>(c / panel_chunks);
    const int ipp = min(4, ki - 4 * p);
    const int64_t tile = (c - p * panel_chunks) >> 7;  // rb * ipp + j
    const int64_t rb = tile / ipp;
    const int i = 4 * p + static_cast<int>(tile - rb * ipp);
    const int64_t row = rb * 16 + (l & 15);
    const int64_t src = row * k + i * 128 + h * 64 + (l >> 4) * 16;
    *reinterpret_cast<uint4*>(out + c * 16) = *reinterpret_cast<const uint4*>(qw + src);
  }
}

}  // namespace tokgroup

hipError_t launch_tile_weights(const uint8_t* qw, int64_t n, int64_t k, uint8_t* out,
                               hipStream_t stream) {
  if (n == 0) return hipSuccess;
  if (n % 16 != 0 || k % 128 != 0) return hipErrorInvalidValue;
  const int64_t chunks = n * k / 16;
  int64_t blocks = (chunks + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  tokgroup::tile_weights_kernel<<<dim3(static_cast<uint32_t>(blocks)), dim3(256), 0,
                                  stream>>>(qw, chunks, n, static_cast<int>(k), out);
  return hipGetLastError();
}

namespace {

// Items sorted longest K first (the deal in rounds relies on it), their
// units numbered in that order, and the launch at the token count's T.
hipError_t launch_items(tokgroup::Item* list, int count, int64_t m, hipStream_t stream) {
  using namespace tokgroup;
  std::stable_sort(list, list + count,
                   [](const Item& p, const Item& q) { return p.k > q.k; });
  Args a{};
  a.count = count;
  a.m = static_cast<int>(m);
  int64_t units = 0;
  for (int i = 0; i < count; ++i) {
    a.it[i] = list[i];
    a.it[i].u0 = static_cast<int>(units);
    units += list[i].n / 64;
  }
  if (units <= 0 || units > (int64_t{1} << 30)) return hipErrorInvalidValue;
  a.units = static_cast<int>(units);
  switch ((m + 15) / 16) {
    case 1: return launch_t<1>(a, stream);
    case 2: return launch_t<2>(a, stream);
    case 3: return launch_t<3>(a, stream);
    case 4: return launch_t<4>(a, stream);
    case 5: case 6: case 7: case 8: return launch_t<8>(a, stream);
    default: return launch_t<16>(a, stream);
  }
}

tokgroup::Item whole_item(const TokLinear& L) {
  return tokgroup::Item{L.qx, L.sx, L.qw, L.sw, L.y, nullptr, static_cast<int>(L.n),
                        static_cast<int>(L.k), static_cast<int>(L.k), 0,
                        static_cast<int>(L.k / 128), 0};
}

bool item_ok(const TokLinear& L) {
  return L.n % 64 == 0 && L.n > 0 && L.k % 128 == 0 && L.k > 0 && L.k <= kTokGroupMaxK;
}

}  // namespace

hipError_t launch_tok_group(const TokLinear* items, int count, int64_t m,
                            hipStream_t stream) {
  using namespace tokgroup;
  if (count < 1 || count > kGroupMax || m < 1 || m > kTokGroupMaxM)
    return hipErrorInvalidValue;
  Item list[kGroupMax];
  for (int i = 0; i < count; ++i) {
    if (!item_ok(items[i])) return hipErrorInvalidValue;
    list[i] = whole_item(items[i]);
  }
  return launch_items(list, count, m, stream);
}

int tok_group_splits(const TokLinear* items, int count, int64_t m, int rq) {
  (void)m;
  if (count < 1 || count > kGroupMax || rq < 0 || rq >= count) return 1;
  int64_t others = 0;
  int64_t k_other = 0;  // the longest K among the other items
  for (int i = 0; i < count; ++i)
    if (i != rq) {
      others += items[i].n / 64;
      k_other = std::max<int64_t>(k_other, items[i].k);
    }
  const int64_t ur = items[rq].n / 64;
  const int kt = static_cast<int>(items[rq].k / 128);
  const int room = count - 1;  // items left for the K ranges
  int best = 1;
  // K ranges of whole 512-byte stages.  Beside other items: the most ranges
  // that are no shorter than the longest other item, so that the item's
  // units are not the launch's long pole (measured on the 36-layer stack at
  // 64 tokens, down with K = 12288 beside k and v, K = 4096: 3 ranges took
  // 55.2 us per layer, 2 / 4 / 6 ranges 58.9 / 60.0 / 60.4 us; and on the
  // decode layer at a few tokens, down beside the six other Linears).  On
  // its own: the most ranges that keep the launch at one workgroup per CU
  // (256 CUs).
  for (int s = 2; s <= kTokGroupMaxSplits && s <= kGroupMax - room; ++s) {
    if (kt % (4 * s) != 0) continue;
    if (count > 1 ? items[rq].k / s >= k_other : others + s * ur <= 256) best = s;
  }
  if (const char* e = test_hook("FP8W8A8_TOKG_SPLITS")) {
    const int v = std::atoi(e);
    if (v >= 1 && v <= kTokGroupMaxSplits && v <= kGroupMax - room && kt % v == 0) best = v;
  }
  return best;
}

hipError_t launch_tok_group_requant(const TokLinear* items, int count, int64_t m, int rq,
                                    int splits, float* part, uint8_t* qy, float* y_scale,
                                    hipStream_t stream) {
  using namespace tokgroup;
  if (count < 1 || count > kGroupMax || m < 1 || m > kTokGroupMaxM || rq < 0 ||
      rq >= count || splits < 1 || count - 1 + splits > kGroupMax)
    return hipErrorInvalidValue;
  const TokLinear& R = items[rq];
  if (!item_ok(R) || R.n > (qy != nullptr ? kRequantMaxN : kTokSplitMaxN) ||
      R.k % (128 * splits) != 0)
    return hipErrorInvalidValue;
  Item list[kGroupMax];
  int c = 0;
  for (int i = 0; i < count; ++i) {
    if (i == rq) continue;
    if (!item_ok(items[i])) return hipErrorInvalidValue;
    list[c++] = whole_item(items[i]);
  }
  // K range j of the re-quantized Linear: codes from byte j * ks of each
  // token row, the tiles from K block j * ks / 128 on, raw sums into part[j].
  const int64_t ks = R.k / splits;
  for (int j = 0; j < splits; ++j)
    list[c++] = Item{R.qx + j * ks, R.sx, R.qw, R.sw, R.y, part + j * m * R.n,
                     static_cast<int>(R.n), static_cast<int>(ks), static_cast<int>(R.k),
                     static_cast<int>(j * ks / 128), static_cast<int>(R.k / 128), 0};
  hipError_t e = launch_items(list, c, m, stream);
  if (e != hipSuccess) return e;
  if (qy == nullptr) return launch_splitk_reduce(part, splits, R.sx, R.sw, m, R.n, R.y, R.n, stream);
  return launch_splitk_reduce_quant(part, splits, R.sx, R.sw, m, R.n, R.y, R.n, qy,
                                    y_scale, stream);
}

}  // namespace fp8w8a8
