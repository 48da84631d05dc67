// C ABI of the FP8_DYNAMIC W8A8 Linear: argument validation, the gfx950
// device check and the choice between the decode (M <= 16) and prefill
// kernels.  Nothing here allocates, frees or synchronizes device memory.
#include "../../include/fp8w8a8.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "launch.h"

namespace {

using fp8w8a8::kGemvMaxM;

thread_local int g_last_hip_error = 0;

constexpr int kMaxDevices = 64;
std::atomic<int> g_device_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

int fail_hip(hipError_t e) {
  g_last_hip_error = static_cast<int>(e);
  return FP8W8A8_ERR_HIP;
}

int check_device() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0) {
    g_last_hip_error = static_cast<int>(e);
    return FP8W8A8_ERR_DEVICE;
  }
  if (dev < kMaxDevices) {
    const int st = g_device_state[dev].load(std::memory_order_relaxed);
    if (st == 1) return FP8W8A8_OK;
    if (st == 2) return FP8W8A8_ERR_DEVICE;
  }
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) {
    g_last_hip_error = static_cast<int>(e);
    return FP8W8A8_ERR_DEVICE;
  }
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < kMaxDevices)
    g_device_state[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? FP8W8A8_OK : FP8W8A8_ERR_DEVICE;
}

bool aligned16(const void* p) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

// Byte range of a [rows, cols] matrix with row stride ld.  Computed in
// 128-bit arithmetic and saturated at the top of the address space, so an
// absurd size can only make the overlap tests below more conservative,
// never wrap around and slip past them.
Range span(const void* p, int64_t rows, int64_t cols, int64_t ld,
           size_t elem) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  if (rows <= 0 || cols <= 0) return Range{lo, lo};
  using u128 = unsigned __int128;
  const u128 hi = static_cast<u128>(lo) +
                  (static_cast<u128>(rows - 1) * static_cast<u128>(ld) +
                   static_cast<u128>(cols)) * elem;
  const u128 top = static_cast<u128>(UINTPTR_MAX);
  return Range{lo, static_cast<uintptr_t>(hi > top ? top : hi)};
}

bool overlap(Range a, Range b) {
  return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi;
}

// Sizes are kept below 2^31 per dimension so that kernels can index rows
// with 32-bit integers; element offsets use 64-bit arithmetic.
constexpr int64_t kMaxDim = (int64_t{1} << 31) - 1;

// A row stride (in elements) for rows of `cols` elements: at least cols, at
// most kMaxDim (so that the byte ranges below cannot wrap), a multiple of 8
// (16-byte aligned rows of 2-byte elements).
bool ld_ok(int64_t ld, int64_t cols) {
  return ld >= cols && ld <= kMaxDim && ld % 8 == 0;
}

int check_quant_args(const uint16_t* src, int64_t rows, int64_t k, int64_t ld,
                     const uint8_t* q, const float* scale) {
  if (!src || !q || !scale) return FP8W8A8_ERR_NULL;
  if (rows < 0 || rows > kMaxDim || k < 1 || k > kMaxDim || k % 8 != 0 ||
      !ld_ok(ld, k))
    return FP8W8A8_ERR_SHAPE;
  if (!aligned16(src) || !aligned16(q) ||
      (reinterpret_cast<uintptr_t>(scale) & 3u) != 0)
    return FP8W8A8_ERR_ALIGN;
  const Range in = span(src, rows, k, ld, 2);
  const Range rq = span(q, rows, k, k, 1);
  const Range rs = span(scale, rows, 1, 1, 4);
  if (overlap(in, rq) || overlap(in, rs) || overlap(rq, rs))
    return FP8W8A8_ERR_ALIAS;
  return FP8W8A8_OK;
}

// The matmul kernels address a tile's rows with 32-bit buffer offsets
// (up to 256 rows x k bytes per descriptor), which bounds k.
constexpr int64_t kMaxLinearK = int64_t{1} << 22;

int check_linear_shape(int64_t m, int64_t n, int64_t k, int64_t ldy) {
  if (m < 0 || m > kMaxDim || n < 0 || n > kMaxDim || n % 16 != 0 ||
      k < 128 || k > kMaxLinearK || k % 128 != 0 || !ld_ok(ldy, n))
    return FP8W8A8_ERR_SHAPE;
  return FP8W8A8_OK;
}

enum class Path { kGemv, kGemvTok, kGemm };

// Decode-sized inputs stream the weights through the K-class MFMA GEMV
// (m <= 4; it can also run up to 16); from 5 to 16 tokens, and up to 32 for
// weight matrices up to 16 MiB, the token-group GEMV is faster (measured on
// the layer's shapes: e.g. one layer at m = 16 in 108.6 us against 130.4;
// beyond that each of its workgroups re-reading all activation codes costs
// too much); everything else takes the tiled MFMA GEMM.
// With the test hooks on, FP8W8A8_FORCE_PATH=gemm|gemv|tok overrides the
// choice (each only within its range of m) so that the kernels can be
// cross-checked on identical inputs.
Path choose_path(int64_t m, int64_t n, int64_t k) {
  const char* force = fp8w8a8::test_hook("FP8W8A8_FORCE_PATH");
  if (force && std::strcmp(force, "gemm") == 0) return Path::kGemm;
  if (force && std::strcmp(force, "gemv") == 0 && m <= kGemvMaxM)
    return Path::kGemv;
  if (force && std::strcmp(force, "tok") == 0 && m <= fp8w8a8::kGemvTokMaxM)
    return Path::kGemvTok;
  if (m <= 4) return Path::kGemv;
  if (m <= kGemvMaxM || (m <= 32 && n * k <= (int64_t{1} << 24)))
    return Path::kGemvTok;
  return Path::kGemm;
}

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Workspace (no state survives a call): a fused call that quantizes in a
// separate kernel before the linear kernel keeps the quantized activations
// [m, k] and their scales [m] there; a GEMM whose plan splits K keeps its
// float32 partial sums [splits, m, n] there.
struct Layout {
  size_t qx = 0, sx = 0, part = 0, total = 0;
};

// What precedes the matmul inside one call: nothing (codes given), the
// per-token quantizer, or the RMSNorm / SiLU-gated activation with it.
enum class Pre { kNone = 0, kQuant = 1, kRmsNorm = 2, kSwiGlu = 3 };

// Whether the decode GEMV does the pre-step in its own staging (no
// workspace for codes).
bool pre_in_gemv(Pre pre, int64_t m, int64_t n, int64_t k) {
  switch (pre) {
    case Pre::kQuant: return fp8w8a8::gemv_fused_fits(m, n, k);
    case Pre::kRmsNorm: return fp8w8a8::gemv_pre_fits(fp8w8a8::kPreRmsNorm, m, n, k);
    case Pre::kSwiGlu: return fp8w8a8::gemv_pre_fits(fp8w8a8::kPreSwiGlu, m, n, k);
    default: return false;
  }
}

// The linear kernel for `path` on staged codes (defined below).
hipError_t linear_on_codes(Path path, const fp8w8a8::GemmPlan& plan,
                           const uint8_t* qx, const float* sx, const uint8_t* qw,
                           const float* w_scale, int64_t m, int64_t n, int64_t k,
                           uint16_t* y, int64_t ldy, float* part, hipStream_t s);

Layout layout_for(int64_t m, int64_t n, int64_t k, Pre pre, Path path,
                  const fp8w8a8::GemmPlan& plan) {
  Layout L;
  if (m == 0 || n == 0) return L;
  if (pre != Pre::kNone && !(path == Path::kGemv && pre_in_gemv(pre, m, n, k))) {
    L.qx = 0;
    L.sx = round_up(static_cast<size_t>(m) * k, 256);
    L.total = L.sx + round_up(static_cast<size_t>(m) * 4, 256);
  }
  if (path == Path::kGemm) {
    const size_t pb = fp8w8a8::gemm_partial_bytes(plan, m, n);
    if (pb > 0) {
      L.part = L.total;
      L.total += round_up(pb, 256);
    }
  }
  return L;
}

}  // namespace

namespace fp8w8a8 {

const char* test_hook(const char* name) {
  static std::once_flag once;
  static bool enabled = false;
  std::call_once(once, [] {
    const char* e = std::getenv("FP8W8A8_TEST_HOOKS");
    enabled = e != nullptr && std::strcmp(e, "1") == 0;
  });
  return enabled ? std::getenv(name) : nullptr;
}

}  // namespace fp8w8a8

namespace {

// ---- The allocation-free variant of the fused forward -----------------------
//
// fp8w8a8_quant_linear_noalloc takes no workspace: where the fused call
// stages the quantized activations (and, for split-K plans, the float32
// partial sums) it uses this file-scope device array instead.  Each GPU
// holds its own copy (allocated when the code object is loaded on that GPU,
// held until the process ends).  Host code never passes the array's name to
// a kernel or a copy -- on the host that name is only a stand-in for the
// symbol -- but the device address that hipGetSymbolAddress returns for the
// current device, looked up once per device and kept in g_scratch_addr.
// Nothing in it has to start at zero: every byte a call's kernels read was
// written earlier in the same call (quantizer before matmul, every split
// before the reduction).  Calls that overlap on one GPU share the array and
// race.
constexpr size_t kNoAllocScratchBytes = size_t{64} << 20;
static_assert(kNoAllocScratchBytes == FP8W8A8_NOALLOC_SCRATCH_BYTES,
              "header and library agree on the scratch size");
__device__ __align__(256) static uint8_t scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices];  // guarded by g_scratch_mu

// The current device's address of `scratch`, looked up on first use with
// that device current.
int scratch_address(uint8_t** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    g_last_hip_error = static_cast<int>(e);
    return FP8W8A8_ERR_DEVICE;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return fail_hip(e);
    if (p == nullptr) return fail_hip(hipErrorInvalidSymbol);
    g_scratch_addr[dev] = p;
  }
  *out = static_cast<uint8_t*>(g_scratch_addr[dev]);
  return FP8W8A8_OK;
}

// The fused forward on a caller workspace (use_scratch == false) or on the
// library's per-device scratch (use_scratch == true, workspace_bytes = its
// size; the workspace pointer is ignored).
int quant_linear_impl(const uint16_t* x, int64_t ldx, const uint8_t* qw,
                      const float* w_scale, int64_t m, int64_t n, int64_t k,
                      uint16_t* y, int64_t ldy, uint8_t* workspace,
                      size_t workspace_bytes, bool use_scratch, void* stream) {
  if (!x || !qw || !w_scale || !y) return FP8W8A8_ERR_NULL;
  int st = check_linear_shape(m, n, k, ldy);
  if (st != FP8W8A8_OK) return st;
  if (!ld_ok(ldx, k)) return FP8W8A8_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(qw) || !aligned16(w_scale) ||
      !aligned16(y) || (!use_scratch && workspace && !aligned16(workspace)))
    return FP8W8A8_ERR_ALIGN;
  const Range ry = span(y, m, n, ldy, 2);
  const Range rx = span(x, m, k, ldx, 2);
  if (overlap(ry, rx) || overlap(ry, span(qw, n, k, k, 1)) ||
      overlap(ry, span(w_scale, n, 1, 1, 4)))
    return FP8W8A8_ERR_ALIAS;
  const Path path = choose_path(m, n, k);
  const fp8w8a8::GemmPlan plan = fp8w8a8::plan_gemm(m, n, k);
  const Layout L = layout_for(m, n, k, Pre::kQuant, path, plan);
  const size_t need = L.total;
  if (need > 0) {
    if (use_scratch) {
      if (need > workspace_bytes) return FP8W8A8_ERR_WORKSPACE;
    } else {
      if (!workspace || workspace_bytes < need) return FP8W8A8_ERR_WORKSPACE;
      const Range rw{reinterpret_cast<uintptr_t>(workspace),
                     reinterpret_cast<uintptr_t>(workspace) + need};
      if (overlap(rw, ry) || overlap(rw, rx) || overlap(rw, span(qw, n, k, k, 1)) ||
          overlap(rw, span(w_scale, n, 1, 1, 4)))
        return FP8W8A8_ERR_ALIAS;
    }
  }
  if (m == 0 || n == 0) return FP8W8A8_OK;
  if ((st = check_device()) != FP8W8A8_OK) return st;
  uint8_t* ws = workspace;
  if (use_scratch) {
    ws = nullptr;
    if (need > 0 && (st = scratch_address(&ws)) != FP8W8A8_OK) return st;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (path == Path::kGemv && fp8w8a8::gemv_fused_fits(m, n, k)) {
    e = fp8w8a8::launch_gemv(x, ldx, nullptr, nullptr, qw, w_scale, m, n, k,
                             y, ldy, s);
  } else {
    // Quantize into the workspace, then run the matching linear kernel.
    uint8_t* qx = ws + L.qx;
    float* sx = reinterpret_cast<float*>(ws + L.sx);
    e = fp8w8a8::launch_quant_rows(x, m, k, ldx, qx, sx, s);
    if (e == hipSuccess) {
      if (path == Path::kGemv)
        e = fp8w8a8::launch_gemv(nullptr, 0, qx, sx, qw, w_scale, m, n, k, y,
                                 ldy, s);
      else if (path == Path::kGemvTok)
        e = fp8w8a8::launch_gemv_tok(qx, sx, qw, w_scale, m, n, k, y, ldy, s);
      else
        e = fp8w8a8::launch_gemm(plan, qx, sx, qw, w_scale, m, n, k, y, ldy,
                                 reinterpret_cast<float*>(ws + L.part), s);
    }
  }
  return e == hipSuccess ? FP8W8A8_OK : fail_hip(e);
}

}  // namespace

namespace {

// Shared validation of fp8w8a8_fp8_linear_group's items (also the items of
// the re-quantizing variant): shapes, alignment and the overlap of every
// output with every input and with the other outputs.
int check_group_items(const fp8w8a8_group_fp8_linear* items, int count, int64_t m,
                      fp8w8a8::TokLinear* g) {
  if (!items) return FP8W8A8_ERR_NULL;
  if (count < 1 || count > fp8w8a8::kGroupMax || m < 1 || m > fp8w8a8::kTokGroupMaxM)
    return FP8W8A8_ERR_SHAPE;
  for (int i = 0; i < count; ++i) {
    const fp8w8a8_group_fp8_linear& L = items[i];
    if (!L.qx || !L.x_scale || !L.qw_tiled || !L.w_scale || !L.y) return FP8W8A8_ERR_NULL;
    // (m * n <= 2^30: the kernel addresses an item's bf16 outputs with
    // 32-bit byte offsets.)
    if (L.n < 64 || L.n > (int64_t{1} << 24) || L.n % 64 != 0 || L.k < 128 ||
        L.k > fp8w8a8::kTokGroupMaxK || L.k % 128 != 0 || L.n * m > (int64_t{1} << 30))
      return FP8W8A8_ERR_SHAPE;
    if (!aligned16(L.qx) || !aligned16(L.x_scale) || !aligned16(L.qw_tiled) ||
        !aligned16(L.w_scale) || !aligned16(L.y))
      return FP8W8A8_ERR_ALIGN;
    g[i] = fp8w8a8::TokLinear{L.qx, L.x_scale, L.qw_tiled, L.w_scale, L.y, L.n, L.k};
  }
  for (int i = 0; i < count; ++i) {
    const Range ry = span(items[i].y, m, items[i].n, items[i].n, 2);
    for (int j = 0; j < count; ++j) {
      const fp8w8a8_group_fp8_linear& L = items[j];
      if (overlap(ry, span(L.qx, m, L.k, L.k, 1)) ||
          overlap(ry, span(L.x_scale, m, 1, 1, 4)) ||
          overlap(ry, span(L.qw_tiled, L.n, L.k, L.k, 1)) ||
          overlap(ry, span(L.w_scale, L.n, 1, 1, 4)) ||
          (j != i && overlap(ry, span(L.y, m, L.n, L.n, 2))))
        return FP8W8A8_ERR_ALIAS;
    }
  }
  return FP8W8A8_OK;
}

// Shape rules of the split item (n <= kRequantMaxN when its output is
// re-quantized); its split count and workspace.
int group_requant_plan(const fp8w8a8_group_fp8_linear* items, int count, int64_t m,
                       int rq, bool requant, fp8w8a8::TokLinear* g, int* splits,
                       size_t* bytes) {
  int st = check_group_items(items, count, m, g);
  if (st != FP8W8A8_OK) return st;
  if (rq < 0 || rq >= count ||
      items[rq].n > (requant ? fp8w8a8::kRequantMaxN : fp8w8a8::kTokSplitMaxN))
    return FP8W8A8_ERR_SHAPE;
  *splits = fp8w8a8::tok_group_splits(g, count, m, rq);
  *bytes = static_cast<size_t>(*splits) * static_cast<size_t>(m) *
           static_cast<size_t>(items[rq].n) * sizeof(float);
  return FP8W8A8_OK;
}

}  // namespace

namespace {

bool kv_group_ok(int64_t width, int64_t group) {
  return group >= 8 && group <= 512 && (group & (group - 1)) == 0 &&
         width % group == 0;
}

}  // namespace

extern "C" {

const char* fp8w8a8_status_string(int status) {
  switch (status) {
    case FP8W8A8_OK: return "FP8W8A8_OK";
    case FP8W8A8_ERR_NULL: return "FP8W8A8_ERR_NULL: a required pointer is NULL";
    case FP8W8A8_ERR_SHAPE: return "FP8W8A8_ERR_SHAPE: a size or stride is out of range";
    case FP8W8A8_ERR_ALIGN: return "FP8W8A8_ERR_ALIGN: a pointer is not 16-byte aligned";
    case FP8W8A8_ERR_ALIAS: return "FP8W8A8_ERR_ALIAS: an output overlaps another buffer";
    case FP8W8A8_ERR_WORKSPACE: return "FP8W8A8_ERR_WORKSPACE: workspace missing or too small";
    case FP8W8A8_ERR_DEVICE: return "FP8W8A8_ERR_DEVICE: no HIP device or not gfx950";
    case FP8W8A8_ERR_HIP: return "FP8W8A8_ERR_HIP: a HIP call or kernel launch failed";
    default: return "FP8W8A8: unknown status";
  }
}

int fp8w8a8_last_hip_error(void) { return g_last_hip_error; }

int fp8w8a8_quantize_weight_channelwise(const uint16_t* w, int64_t n,
                                        int64_t k, int64_t ldw, uint8_t* qw,
                                        float* w_scale, void* stream) {
  int st = check_quant_args(w, n, k, ldw, qw, w_scale);
  if (st != FP8W8A8_OK) return st;
  if (n == 0) return FP8W8A8_OK;
  if ((st = check_device()) != FP8W8A8_OK) return st;
  hipError_t e = fp8w8a8::launch_quant_rows(w, n, k, ldw, qw, w_scale,
                                            static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8W8A8_OK : fail_hip(e);
}

int fp8w8a8_quantize_act_per_token(const uint16_t* x, int64_t m, int64_t k,
                                   int64_t ldx, uint8_t* qx, float* x_scale,
                                   void* stream) {
  int st = check_quant_args(x, m, k, ldx, qx, x_scale);
  if (st != FP8W8A8_OK) return st;
  if (m == 0) return FP8W8A8_OK;
  if ((st = check_device()) != FP8W8A8_OK) return st;
  hipError_t e = fp8w8a8::launch_quant_rows(x, m, k, ldx, qx, x_scale,
                                            static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8W8A8_OK : fail_hip(e);
}

int fp8w8a8_rmsnorm_quantize(const uint16_t* x, int64_t m, int64_t k,
                             int64_t ldx, const uint16_t* gamma, float eps,
                             uint8_t* qx, float* x_scale, uint16_t* y,
                             int64_t ldy, void* stream) {
  if (!x || !gamma || !qx || !x_scale) return FP8W8A8_ERR_NULL;
  if (m < 0 || m > kMaxDim || k < 8 || k > kMaxDim || k % 8 != 0 ||
      !ld_ok(ldx, k) || (y && !ld_ok(ldy, k)) ||
      !(eps >= 0.0f && eps <= 3.4028235e38f))
    return FP8W8A8_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(gamma) || !aligned16(qx) ||
      (y && !aligned16(y)) || (reinterpret_cast<uintptr_t>(x_scale) & 3u) != 0)
    return FP8W8A8_ERR_ALIGN;
  const Range rx = span(x, m, k, ldx, 2);
  const Range rg = span(gamma, 1, k, k, 2);
  const Range rq = span(qx, m, k, k, 1);
  const Range rs = span(x_scale, m, 1, 1, 4);
  const Range ry = y ? span(y, m, k, ldy, 2) : Range{0, 0};
  const Range outs[3] = {rq, rs, ry};
  for (int i = 0; i < 3; ++i) {
    if (overlap(outs[i], rx) || overlap(outs[i], rg)) return FP8W8A8_ERR_ALIAS;
    for (int j = i + 1; j < 3; ++j)
      if (overlap(outs[i], outs[j])) return FP8W8A8_ERR_ALIAS;
  }
  if (m == 0) return FP8W8A8_OK;
  int st = check_device();
  if (st != FP8W8A8_OK) return st;
  hipError_t e = fp8w8a8::launch_rmsnorm_quant(
      x, m, k, ldx, gamma, eps, qx, x_scale, y, ldy,
      static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8W8A8_OK : fail_hip(e);
}

int fp8w8a8_swiglu_quantize(const uint16_t* gate, int64_t ldg,
                            const uint16_t* up, int64_t ldu, int64_t m,
                            int64_t n, uint8_t* qh, float* h_scale,
                            uint16_t* h, int64_t ldh, void* stream) {
  if (!gate || !up || !qh || !h_scale) return FP8W8A8_ERR_NULL;
  if (m < 0 || m > kMaxDim || n < 8 || n > kMaxDim || n % 8 != 0 ||
      !ld_ok(ldg, n) || !ld_ok(ldu, n) || (h && !ld_ok(ldh, n)))
    return FP8W8A8_ERR_SHAPE;
  if (!aligned16(gate) || !aligned16(up) || !aligned16(qh) || (h && !aligned16(h)) ||
      (reinterpret_cast<uintptr_t>(h_scale) & 3u) != 0)
    return FP8W8A8_ERR_ALIGN;
  const Range rg = span(gate, m, n, ldg, 2);
  const Range ru = span(up, m, n, ldu, 2);
  const Range outs[3] = {span(qh, m, n, n, 1), span(h_scale, m, 1, 1, 4),
                         h ? span(h, m, n, ldh, 2) : Range{0, 0}};
  for (int i = 0; i < 3; ++i) {
    if (overlap(outs[i], rg) || overlap(outs[i], ru)) return FP8W8A8_ERR_ALIAS;
    for (int j = i + 1; j < 3; ++j)
      if (overlap(outs[i], outs[j])) return FP8W8A8_ERR_ALIAS;
  }
  if (m == 0) return FP8W8A8_OK;
  int st = check_device();
  if (st != FP8W8A8_OK) return st;
  hipError_t e = fp8w8a8::launch_swiglu_quant(gate, ldg, up, ldu, m, n, qh,
                                              h_scale, h, ldh,
                                              static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8W8A8_OK : fail_hip(e);
}

int fp8w8a8_kv_quantize_fp8(const uint16_t* kv, int64_t rows, int64_t width,
                            int64_t ld, int64_t group, uint8_t* codes,
                            float* scales, void* stream) {
  if (!kv || !codes || !scales) return FP8W8A8_ERR_NULL;
  if (rows < 0 || rows > kMaxDim || width < 8 || width > kMaxDim ||
      width % 8 != 0 || !kv_group_ok(width, group) || !ld_ok(ld, width))
    return FP8W8A8_ERR_SHAPE;
  if (!aligned16(kv) || (reinterpret_cast<uintptr_t>(codes) & 7u) != 0 ||
      (reinterpret_cast<uintptr_t>(scales) & 3u) != 0)
    return FP8W8A8_ERR_ALIGN;
  const Range rx = span(kv, rows, width, ld, 2);
  const Range rc = span(codes, rows, width, width, 1);
  const Range rs = span(scales, rows, width / group, width / group, 4);
  if (overlap(rc, rx) || overlap(rs, rx) || overlap(rc, rs)) return FP8W8A8_ERR_ALIAS;
  if (rows == 0) return FP8W8A8_OK;
  int st = check_device();
  if (st != FP8W8A8_OK) return st;
  hipError_t e = fp8w8a8::launch_kv_quantize(kv, rows, width, ld, group, codes,
                                             scales, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8W8A8_OK : fail_hip(e);
}

int fp8w8a8_kv_dequantize_fp8(const uint8_t* codes, const float* scales,
                              int64_t rows, int64_t width, int64_t group,
                              uint16_t* out, int64_t ldo, void* stream) {
  if (!codes || !scales || !out) return FP8W8A8_ERR_NULL;
  if (rows < 0 || rows > kMaxDim || width < 8 || width > kMaxDim ||
      width % 8 != 0 || !kv_group_ok(width, group) || !ld_ok(ldo, width))
    return FP8W8A8_ERR_SHAPE;
  if (!aligned16(out) || (reinterpret_cast<uintptr_t>(codes) & 7u) != 0 ||
      (reinterpret_cast<uintptr_t>(scales) & 3u) != 0)
    return FP8W8A8_ERR_ALIGN;
  const Range ro = span(out, rows, width, ldo, 2);
  if (overlap(ro, span(codes, rows, width, width, 1)) ||
      overlap(ro, span(scales, rows, width / group, width / group, 4)))
    return FP8W8A8_ERR_ALIAS;
  if (rows == 0) return FP8W8A8_OK;
  int st = check_device();
  if (st != FP8W8A8_OK) return st;
  hipError_t e = fp8w8a8::launch_kv_dequantize(codes, scales, rows, width, group,
                                               out, ldo, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8W8A8_OK : fail_hip(e);
}

int fp8w8a8_kv_quantize_int8(const uint16_t* kv, int64_t rows, int64_t width,
                             int64_t ld, int64_t group, uint8_t* codes,
                             float* scales, float* mins, void* stream) {
  if (!kv || !codes || !scales || !mins) return FP8W8A8_ERR_NULL;
  if (rows < 0 || rows > kMaxDim || width < 8 || width > kMaxDim ||
      width % 8 != 0 || !kv_group_ok(width, group) || !ld_ok(ld, width))
    return FP8W8A8_ERR_SHAPE;
  if (!aligned16(kv) || (reinterpret_cast<uintptr_t>(codes) & 7u) != 0 ||
      (reinterpret_cast<uintptr_t>(scales) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(mins) & 3u) != 0)
    return FP8W8A8_ERR_ALIGN;
  const int64_t g = width / group;
  const Range rx = span(kv, rows, width, ld, 2);
  const Range outs[3] = {span(codes, rows, width, width, 1), span(scales, rows, g, g, 4),
                         span(mins, rows, g, g, 4)};
  for (int i = 0; i < 3; ++i) {
    if (overlap(outs[i], rx)) return FP8W8A8_ERR_ALIAS;
    for (int j = i + 1; j < 3; ++j)
      if (overlap(outs[i], outs[j])) return FP8W8A8_ERR_ALIAS;
  }
  if (rows == 0) return FP8W8A8_OK;
  int st = check_device();
  if (st != FP8W8A8_OK) return st;
  hipError_t e = fp8w8a8::launch_kv_quantize_int8(kv, rows, width, ld, group, codes,
                                                  scales, mins,
                                                  static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8W8A8_OK : fail_hip(e);
}

int fp8w8a8_kv_read_int8(const uint8_t* codes, const float* scales,
                         const float* mins, int64_t hist,
                         const uint16_t* tail, int64_t tail_rows, int64_t ldt,
                         int64_t width, int64_t group, uint16_t* out,
                         int64_t ldo, void* stream) {
  if (!out || (hist > 0 && (!codes || !scales || !mins)) || (tail_rows > 0 && !tail))
    return FP8W8A8_ERR_NULL;
  if (hist < 0 || tail_rows < 0 || hist > kMaxDim || tail_rows > kMaxDim ||
      hist + tail_rows > kMaxDim || width < 8 || width > kMaxDim || width % 8 != 0 ||
      !kv_group_ok(width, group) || !ld_ok(ldo, width) ||
      (tail_rows > 0 && !ld_ok(ldt, width)))
    return FP8W8A8_ERR_SHAPE;
  if (!aligned16(out) || (tail_rows > 0 && !aligned16(tail)) ||
      (hist > 0 && ((reinterpret_cast<uintptr_t>(codes) & 7u) != 0 ||
                    (reinterpret_cast<uintptr_t>(scales) & 3u) != 0 ||
                    (reinterpret_cast<uintptr_t>(mins) & 3u) != 0)))
    return FP8W8A8_ERR_ALIGN;
  const int64_t g = width / group;
  const Range ro = span(out, hist + tail_rows, width, ldo, 2);
  if (overlap(ro, span(codes, hist, width, width, 1)) ||
      overlap(ro, span(scales, hist, g, g, 4)) || overlap(ro, span(mins, hist, g, g, 4)) ||
      overlap(ro, span(tail, tail_rows, width, ldt, 2)))
    return FP8W8A8_ERR_ALIAS;
  if (hist + tail_rows == 0) return FP8W8A8_OK;
  int st = check_device();
  if (st != FP8W8A8_OK) return st;
  hipError_t e = fp8w8a8::launch_kv_read_int8(codes, scales, mins, hist, tail,
                                              tail_rows, ldt, width, group, out, ldo,
                                              static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8W8A8_OK : fail_hip(e);
}

size_t fp8w8a8_workspace_bytes(int64_t m, int64_t n, int64_t k, int fused) {
  if (check_linear_shape(m, n, k, n) != FP8W8A8_OK) return 0;
  const Pre pre = fused == 0 ? Pre::kNone
                : fused == 2 ? Pre::kRmsNorm
                : fused == 3 ? Pre::kSwiGlu : Pre::kQuant;
  return layout_for(m, n, k, pre, choose_path(m, n, k),
                    fp8w8a8::plan_gemm(m, n, k)).total;
}

int fp8w8a8_fp8_linear(const uint8_t* qx, const float* x_scale,
                       const uint8_t* qw, const float* w_scale, int64_t m,
                       int64_t n, int64_t k, uint16_t* y, int64_t ldy,
                       void* workspace, size_t workspace_bytes, void* stream) {
  if (!qx || !x_scale || !qw || !w_scale || !y) return FP8W8A8_ERR_NULL;
  int st = check_linear_shape(m, n, k, ldy);
  if (st != FP8W8A8_OK) return st;
  if (!aligned16(qx) || !aligned16(x_scale) || !aligned16(qw) ||
      !aligned16(w_scale) || !aligned16(y) ||
      (workspace && !aligned16(workspace)))
    return FP8W8A8_ERR_ALIGN;
  const Range ry = span(y, m, n, ldy, 2);
  if (overlap(ry, span(qx, m, k, k, 1)) || overlap(ry, span(x_scale, m, 1, 1, 4)) ||
      overlap(ry, span(qw, n, k, k, 1)) || overlap(ry, span(w_scale, n, 1, 1, 4)))
    return FP8W8A8_ERR_ALIAS;
  const Path path = choose_path(m, n, k);
  const fp8w8a8::GemmPlan plan = fp8w8a8::plan_gemm(m, n, k);
  const Layout L = layout_for(m, n, k, Pre::kNone, path, plan);
  const size_t need = L.total;
  if (need > 0) {
    if (!workspace || workspace_bytes < need) return FP8W8A8_ERR_WORKSPACE;
    const Range rw{reinterpret_cast<uintptr_t>(workspace),
                   reinterpret_cast<uintptr_t>(workspace) + need};
    if (overlap(rw, ry) || overlap(rw, span(qx, m, k, k, 1)) ||
        overlap(rw, span(qw, n, k, k, 1)) ||
        overlap(rw, span(x_scale, m, 1, 1, 4)) ||
        overlap(rw, span(w_scale, n, 1, 1, 4)))
      return FP8W8A8_ERR_ALIAS;
  }
  if (m == 0 || n == 0) return FP8W8A8_OK;
  if ((st = check_device()) != FP8W8A8_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (path == Path::kGemv)
    e = fp8w8a8::launch_gemv(nullptr, 0, qx, x_scale, qw, w_scale, m, n, k, y,
                             ldy, s);
  else if (path == Path::kGemvTok)
    e = fp8w8a8::launch_gemv_tok(qx, x_scale, qw, w_scale, m, n, k, y, ldy, s);
  else
    e = fp8w8a8::launch_gemm(plan, qx, x_scale, qw, w_scale, m, n, k, y, ldy,
                             reinterpret_cast<float*>(
                                 static_cast<uint8_t*>(workspace) + L.part),
                             s);
  return e == hipSuccess ? FP8W8A8_OK : fail_hip(e);
}

int fp8w8a8_fp8_linear_requant(const uint8_t* qx, const float* x_scale,
                               const uint8_t* qw, const float* w_scale, int64_t m,
                               int64_t n, int64_t k, uint16_t* y, int64_t ldy,
                               uint8_t* qy, float* y_scale, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (!qx || !x_scale || !qw || !w_scale || !y || !qy || !y_scale) return FP8W8A8_ERR_NULL;
  int st = check_linear_shape(m, n, k, ldy);
  if (st != FP8W8A8_OK) return st;
  if (!aligned16(qx) || !aligned16(x_scale) || !aligned16(qw) ||
      !aligned16(w_scale) || !aligned16(y) || !aligned16(qy) ||
      (reinterpret_cast<uintptr_t>(y_scale) & 3u) != 0 ||
      (workspace && !aligned16(workspace)))
    return FP8W8A8_ERR_ALIGN;
  // Outputs: y, its codes and its scales; none may overlap an input or
  // another output.
  const Range outs[3] = {span(y, m, n, ldy, 2), span(qy, m, n, n, 1),
                         span(y_scale, m, 1, 1, 4)};
  const Range ins[4] = {span(qx, m, k, k, 1), span(x_scale, m, 1, 1, 4),
                        span(qw, n, k, k, 1), span(w_scale, n, 1, 1, 4)};
  for (int i = 0; i < 3; ++i) {
    for (const Range& r : ins)
      if (overlap(outs[i], r)) return FP8W8A8_ERR_ALIAS;
    for (int j = i + 1; j < 3; ++j)
      if (overlap(outs[i], outs[j])) return FP8W8A8_ERR_ALIAS;
  }
  const Path path = choose_path(m, n, k);
  const fp8w8a8::GemmPlan plan = fp8w8a8::plan_gemm(m, n, k);
  const Layout L = layout_for(m, n, k, Pre::kNone, path, plan);
  if (L.total > 0) {
    if (!workspace || workspace_bytes < L.total) return FP8W8A8_ERR_WORKSPACE;
    const Range rw{reinterpret_cast<uintptr_t>(workspace),
                   reinterpret_cast<uintptr_t>(workspace) + L.total};
    for (const Range& r : outs)
      if (overlap(rw, r)) return FP8W8A8_ERR_ALIAS;
    for (const Range& r : ins)
      if (overlap(rw, r)) return FP8W8A8_ERR_ALIAS;
  }
  if (m == 0 || n == 0) return FP8W8A8_OK;
  if ((st = check_device()) != FP8W8A8_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* part = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + L.part);
  hipError_t e;
  if (path == Path::kGemm) {
    e = fp8w8a8::launch_gemm_requant(plan, qx, x_scale, qw, w_scale, m, n, k, y, ldy,
                                     qy, y_scale, part, s);
  } else {
    e = linear_on_codes(path, plan, qx, x_scale, qw, w_scale, m, n, k, y, ldy, part, s);
    if (e == hipSuccess) e = fp8w8a8::launch_quant_rows(y, m, n, ldy, qy, y_scale, s);
  }
  return e == hipSuccess ? FP8W8A8_OK : fail_hip(e);
}

int fp8w8a8_quant_linear(const uint16_t* x, int64_t ldx, const uint8_t* qw,
                         const float* w_scale, int64_t m, int64_t n, int64_t k,
                         uint16_t* y, int64_t ldy, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return quant_linear_impl(x, ldx, qw, w_scale, m, n, k, y, ldy,
                           static_cast<uint8_t*>(workspace), workspace_bytes,
                           false, stream);
}

int fp8w8a8_quant_linear_group_m1(const fp8w8a8_group_linear* items, int count,
                                  void* stream) {
  if (!items) return FP8W8A8_ERR_NULL;
  if (count < 1 || count > fp8w8a8::kGroupMax) return FP8W8A8_ERR_SHAPE;
  fp8w8a8::GroupLinear g[fp8w8a8::kGroupMax];
  for (int i = 0; i < count; ++i) {
    const fp8w8a8_group_linear& L = items[i];
    if (!L.x || !L.qw || !L.w_scale || !L.y) return FP8W8A8_ERR_NULL;
    if (L.n < 16 || L.n > kMaxDim || L.n % 16 != 0 || L.k < 128 || L.k > 12288 ||
        L.k % 128 != 0)
      return FP8W8A8_ERR_SHAPE;
    if (!aligned16(L.x) || !aligned16(L.qw) || !aligned16(L.w_scale) || !aligned16(L.y))
      return FP8W8A8_ERR_ALIGN;
    g[i] = fp8w8a8::GroupLinear{L.x, L.qw, L.w_scale, L.y, L.n, L.k};
  }
  for (int i = 0; i < count; ++i) {
    const Range ry = span(items[i].y, 1, items[i].n, items[i].n, 2);
    for (int j = 0; j < count; ++j) {
      const fp8w8a8_group_linear& L = items[j];
      if (overlap(ry, span(L.x, 1, L.k, L.k, 2)) ||
          overlap(ry, span(L.qw, L.n, L.k, L.k, 1)) ||
          overlap(ry, span(L.w_scale, L.n, 1, 1, 4)) ||
          (j != i && overlap(ry, span(L.y, 1, L.n, L.n, 2))))
        return FP8W8A8_ERR_ALIAS;
    }
  }
  int st = check_device();
  if (st != FP8W8A8_OK) return st;
  hipError_t e = fp8w8a8::launch_gemv_group_m1(g, count, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8W8A8_OK : fail_hip(e);
}

int fp8w8a8_quantize_act_group(const fp8w8a8_group_quant* items, int count,
                               void* stream) {
  if (!items) return FP8W8A8_ERR_NULL;
  if (count < 1 || count > fp8w8a8::kGroupMax) return FP8W8A8_ERR_SHAPE;
  fp8w8a8::QuantItem g[fp8w8a8::kGroupMax];
  int live = 0;
  int64_t rows = 0;
  for (int i = 0; i < count; ++i) {
    const fp8w8a8_group_quant& L = items[i];
    if (L.m == 0) {  // nothing to read or write: only the shape is checked
      if (L.k < 8 || L.k > fp8w8a8::kQuantGroupMaxK || L.k % 8 != 0 || !ld_ok(L.ldx, L.k))
        return FP8W8A8_ERR_SHAPE;
      continue;
    }
    const int st = check_quant_args(L.x, L.m, L.k, L.ldx, L.qx, L.x_scale);
    if (st != FP8W8A8_OK) return st;
    if (L.k > fp8w8a8::kQuantGroupMaxK) return FP8W8A8_ERR_SHAPE;
    rows += L.m;
    if (rows > kMaxDim) return FP8W8A8_ERR_SHAPE;
    g[live++] = fp8w8a8::QuantItem{L.x, L.m, L.k, L.ldx, L.qx, L.x_scale, 0};
  }
  // No output may overlap any item's input or another output.
  for (int i = 0; i < count; ++i) {
    const Range oq = span(items[i].qx, items[i].m, items[i].k, items[i].k, 1);
    const Range os = span(items[i].x_scale, items[i].m, 1, 1, 4);
    for (int j = 0; j < count; ++j) {
      const Range in = span(items[j].x, items[j].m, items[j].k, items[j].ldx, 2);
      if (overlap(oq, in) || overlap(os, in)) return FP8W8A8_ERR_ALIAS;
      if (j != i &&
          (overlap(oq, span(items[j].qx, items[j].m, items[j].k, items[j].k, 1)) ||
           overlap(oq, span(items[j].x_scale, items[j].m, 1, 1, 4)) ||
           overlap(os, span(items[j].qx, items[j].m, items[j].k, items[j].k, 1)) ||
           overlap(os, span(items[j].x_scale, items[j].m, 1, 1, 4))))
        return FP8W8A8_ERR_ALIAS;
    }
  }
  if (rows == 0) return FP8W8A8_OK;
  int st = check_device();
  if (st != FP8W8A8_OK) return st;
  hipError_t e = fp8w8a8::launch_quant_group(g, live, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8W8A8_OK : fail_hip(e);
}

int fp8w8a8_tile_weights(const uint8_t* qw, int64_t n, int64_t k, uint8_t* tiled,
                         void* stream) {
  if (!qw || !tiled) return FP8W8A8_ERR_NULL;
  if (n < 0 || n > kMaxDim || n % 16 != 0 || k < 128 || k > fp8w8a8::kTokGroupMaxK ||
      k % 128 != 0)
    return FP8W8A8_ERR_SHAPE;
  if (!aligned16(qw) || !aligned16(tiled)) return FP8W8A8_ERR_ALIGN;
  if (overlap(span(qw, n, k, k, 1), span(tiled, n, k, k, 1))) return FP8W8A8_ERR_ALIAS;
  if (n == 0) return FP8W8A8_OK;
  int st = check_device();
  if (st != FP8W8A8_OK) return st;
  hipError_t e = fp8w8a8::launch_tile_weights(qw, n, k, tiled, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8W8A8_OK : fail_hip(e);
}

int fp8w8a8_fp8_linear_group(const fp8w8a8_group_fp8_linear* items, int count,
                             int64_t m, void* stream) {
  fp8w8a8::TokLinear g[fp8w8a8::kGroupMax];
  int st = check_group_items(items, count, m, g);
  if (st != FP8W8A8_OK) return st;
  if ((st = check_device()) != FP8W8A8_OK) return st;
  hipError_t e = fp8w8a8::launch_tok_group(g, count, m, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8W8A8_OK : fail_hip(e);
}

size_t fp8w8a8_group_requant_workspace_bytes(const fp8w8a8_group_fp8_linear* items,
                                             int count, int64_t m, int rq) {
  fp8w8a8::TokLinear g[fp8w8a8::kGroupMax];
  int splits = 0;
  size_t bytes = 0;
  return group_requant_plan(items, count, m, rq, false, g, &splits, &bytes) == FP8W8A8_OK
             ? bytes
             : 0;
}

int fp8w8a8_fp8_linear_group_requant(const fp8w8a8_group_fp8_linear* items, int count,
                                     int64_t m, int rq, uint8_t* qy, float* y_scale,
                                     void* workspace, size_t workspace_bytes,
                                     void* stream) {
  fp8w8a8::TokLinear g[fp8w8a8::kGroupMax];
  int splits = 0;
  size_t need = 0;
  // qy and y_scale: both given (re-quantize) or both null (split only).
  const bool requant = qy != nullptr || y_scale != nullptr;
  int st = group_requant_plan(items, count, m, rq, requant, g, &splits, &need);
  if (st != FP8W8A8_OK) return st;
  if ((requant && (!qy || !y_scale)) || !workspace) return FP8W8A8_ERR_NULL;
  if ((requant && (!aligned16(qy) || (reinterpret_cast<uintptr_t>(y_scale) & 3u) != 0)) ||
      !aligned16(workspace))
    return FP8W8A8_ERR_ALIGN;
  if (workspace_bytes < need) return FP8W8A8_ERR_WORKSPACE;
  // qy, y_scale and the workspace overlap no input, no y and one another
  // (a null output's range is empty).
  const Range extra[3] = {span(qy, requant ? m : 0, items[rq].n, items[rq].n, 1),
                          span(y_scale, requant ? m : 0, 1, 1, 4),
                          Range{reinterpret_cast<uintptr_t>(workspace),
                                reinterpret_cast<uintptr_t>(workspace) + need}};
  for (int a = 0; a < 3; ++a) {
    for (int b = a + 1; b < 3; ++b)
      if (overlap(extra[a], extra[b])) return FP8W8A8_ERR_ALIAS;
    for (int j = 0; j < count; ++j) {
      const fp8w8a8_group_fp8_linear& L = items[j];
      if (overlap(extra[a], span(L.qx, m, L.k, L.k, 1)) ||
          overlap(extra[a], span(L.x_scale, m, 1, 1, 4)) ||
          overlap(extra[a], span(L.qw_tiled, L.n, L.k, L.k, 1)) ||
          overlap(extra[a], span(L.w_scale, L.n, 1, 1, 4)) ||
          overlap(extra[a], span(L.y, m, L.n, L.n, 2)))
        return FP8W8A8_ERR_ALIAS;
    }
  }
  if ((st = check_device()) != FP8W8A8_OK) return st;
  hipError_t e = fp8w8a8::launch_tok_group_requant(
      g, count, m, rq, splits, static_cast<float*>(workspace), qy, y_scale,
      static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8W8A8_OK : fail_hip(e);
}

int fp8w8a8_quant_linear_noalloc(const uint16_t* x, int64_t ldx,
                                 const uint8_t* qw, const float* w_scale,
                                 int64_t m, int64_t n, int64_t k, uint16_t* y,
                                 int64_t ldy, void* stream) {
  return quant_linear_impl(x, ldx, qw, w_scale, m, n, k, y, ldy, nullptr,
                           kNoAllocScratchBytes, true, stream);
}

}  // extern "C"

namespace {

// The linear kernel for `path` on staged codes (qx, sx).
hipError_t linear_on_codes(Path path, const fp8w8a8::GemmPlan& plan,
                           const uint8_t* qx, const float* sx, const uint8_t* qw,
                           const float* w_scale, int64_t m, int64_t n, int64_t k,
                           uint16_t* y, int64_t ldy, float* part, hipStream_t s) {
  if (path == Path::kGemv)
    return fp8w8a8::launch_gemv(nullptr, 0, qx, sx, qw, w_scale, m, n, k, y, ldy, s);
  if (path == Path::kGemvTok)
    return fp8w8a8::launch_gemv_tok(qx, sx, qw, w_scale, m, n, k, y, ldy, s);
  return fp8w8a8::launch_gemm(plan, qx, sx, qw, w_scale, m, n, k, y, ldy, part, s);
}

// RMSNorm or SiLU-gated activation, then the Linear: x [m, k] (ldx) with
// x2 = gamma [k] (kRmsNorm) or up [m, k] (ld2, kSwiGlu).
int pre_linear(Pre pre, const uint16_t* x, int64_t ldx, const uint16_t* x2,
               int64_t ld2, float eps, const uint8_t* qw, const float* w_scale,
               int64_t m, int64_t n, int64_t k, uint16_t* y, int64_t ldy,
               void* workspace, size_t workspace_bytes, void* stream) {
  if (!x || !x2 || !qw || !w_scale || !y) return FP8W8A8_ERR_NULL;
  int st = check_linear_shape(m, n, k, ldy);
  if (st != FP8W8A8_OK) return st;
  if (!ld_ok(ldx, k)) return FP8W8A8_ERR_SHAPE;
  if (pre == Pre::kSwiGlu && !ld_ok(ld2, k)) return FP8W8A8_ERR_SHAPE;
  if (pre == Pre::kRmsNorm && !(eps >= 0.0f && eps <= 3.4028235e38f))
    return FP8W8A8_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(x2) || !aligned16(qw) || !aligned16(w_scale) ||
      !aligned16(y) || (workspace && !aligned16(workspace)))
    return FP8W8A8_ERR_ALIGN;
  const Range ry = span(y, m, n, ldy, 2);
  const Range rx = span(x, m, k, ldx, 2);
  const Range r2 = pre == Pre::kRmsNorm ? span(x2, 1, k, k, 2) : span(x2, m, k, ld2, 2);
  if (overlap(ry, rx) || overlap(ry, r2) || overlap(ry, span(qw, n, k, k, 1)) ||
      overlap(ry, span(w_scale, n, 1, 1, 4)))
    return FP8W8A8_ERR_ALIAS;
  const Path path = choose_path(m, n, k);
  const fp8w8a8::GemmPlan plan = fp8w8a8::plan_gemm(m, n, k);
  const Layout L = layout_for(m, n, k, pre, path, plan);
  if (L.total > 0) {
    if (!workspace || workspace_bytes < L.total) return FP8W8A8_ERR_WORKSPACE;
    const Range rw{reinterpret_cast<uintptr_t>(workspace),
                   reinterpret_cast<uintptr_t>(workspace) + L.total};
    if (overlap(rw, ry) || overlap(rw, rx) || overlap(rw, r2) ||
        overlap(rw, span(qw, n, k, k, 1)) || overlap(rw, span(w_scale, n, 1, 1, 4)))
      return FP8W8A8_ERR_ALIAS;
  }
  if (m == 0 || n == 0) return FP8W8A8_OK;
  if ((st = check_device()) != FP8W8A8_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int gpre = pre == Pre::kRmsNorm ? fp8w8a8::kPreRmsNorm : fp8w8a8::kPreSwiGlu;
  hipError_t e;
  if (path == Path::kGemv && pre_in_gemv(pre, m, n, k)) {
    e = fp8w8a8::launch_gemv_pre(gpre, x, ldx, x2, ld2, eps, qw, w_scale, m, n, k,
                                 y, ldy, s);
  } else {
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    uint8_t* qx = ws + L.qx;
    float* sx = reinterpret_cast<float*>(ws + L.sx);
    e = pre == Pre::kRmsNorm
            ? fp8w8a8::launch_rmsnorm_quant(x, m, k, ldx, x2, eps, qx, sx, nullptr, 0, s)
            : fp8w8a8::launch_swiglu_quant(x, ldx, x2, ld2, m, k, qx, sx, nullptr, 0, s);
    if (e == hipSuccess)
      e = linear_on_codes(path, plan, qx, sx, qw, w_scale, m, n, k, y, ldy,
                          reinterpret_cast<float*>(ws + L.part), s);
  }
  return e == hipSuccess ? FP8W8A8_OK : fail_hip(e);
}

}  // namespace

extern "C" {

int fp8w8a8_rmsnorm_quant_linear(const uint16_t* x, int64_t ldx,
                                 const uint16_t* gamma, float eps,
                                 const uint8_t* qw, const float* w_scale,
                                 int64_t m, int64_t n, int64_t k, uint16_t* y,
                                 int64_t ldy, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  return pre_linear(Pre::kRmsNorm, x, ldx, gamma, 0, eps, qw, w_scale, m, n, k, y,
                    ldy, workspace, workspace_bytes, stream);
}

int fp8w8a8_swiglu_quant_linear(const uint16_t* gate, int64_t ldg,
                                const uint16_t* up, int64_t ldu,
                                const uint8_t* qw, const float* w_scale,
                                int64_t m, int64_t n, int64_t k, uint16_t* y,
                                int64_t ldy, void* workspace,
                                size_t workspace_bytes, void* stream) {
  return pre_linear(Pre::kSwiGlu, gate, ldg, up, ldu, 0.0f, qw, w_scale, m, n, k, y,
                    ldy, workspace, workspace_bytes, stream);
}

int fp8w8a8_workspace_init(void* workspace, size_t bytes, void* stream) {
  if (!workspace) return FP8W8A8_ERR_NULL;
  if (bytes % 16 != 0) return FP8W8A8_ERR_SHAPE;
  if (!aligned16(workspace)) return FP8W8A8_ERR_ALIGN;
  if (bytes == 0) return FP8W8A8_OK;
  int st = check_device();
  if (st != FP8W8A8_OK) return st;
  hipError_t e = fp8w8a8::launch_zero_fill(workspace, bytes,
                                           static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8W8A8_OK : fail_hip(e);
}

}  // extern "C"
