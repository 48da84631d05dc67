/*
 * fp8w8a8.h — C ABI of the FP8_DYNAMIC W8A8 Linear for AMD Instinct MI355X
 * (gfx950).
 *
 * What the library computes (MOSS-VL quantization README, "FP8-Dynamic"
 * recipe; MOSS-VL-Realtime-FP8 article, section on why the 252 Linears use
 * FP8 E4M3):
 *   - weights are stored as float8_e4m3fn (OCP E4M3: 4 exponent bits,
 *     3 mantissa bits, bias 7, largest finite value 448) with one static
 *     float32 scale per output channel, computed once, offline;
 *   - the Linear's bf16 input is quantized at run time to E4M3 with one
 *     dynamic float32 scale per token (row);
 *   - the Linear multiplies the two FP8 operands, accumulates in float32 and
 *     writes bfloat16: y[m,n] = bf16( sum_k dec(qx[m,k]) * dec(qw[n,k])
 *                                     * x_scale[m] * w_scale[n] ), no bias.
 * Quantization of one row r (token or output channel), where the pages give
 * no formula (readings, stated once here):
 *     amax  = max_k |v[r,k]|
 *     scale = amax / 448            (IEEE float32 division)
 *     code  = e4m3(v[r,k] / scale)  (IEEE float32 division, then round to
 *                                    nearest, ties to even, saturate to
 *                                    +-448, sign kept; amax == 0 gives
 *                                    scale 0 and codes +-0)
 *
 * Conventions for every entry point:
 *   - tensor pointers are DEVICE pointers on the current HIP device;
 *   - all matrices are row-major; ld* are row strides in ELEMENTS;
 *   - bfloat16 values are passed as their uint16_t bit patterns, E4M3 codes
 *     as uint8_t bytes; scales are float32;
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream);
 *     kernels are enqueued on it and the call returns without waiting;
 *   - the caller owns every buffer; the library never allocates, frees or
 *     synchronizes device memory, and keeps only a cache of device facts;
 *   - arguments are validated before anything is enqueued; on a non-zero
 *     status nothing was enqueued and no output was touched, except
 *     FP8W8A8_ERR_HIP from a failed launch (outputs then unspecified);
 *   - M == 0 or N == 0 is a valid empty call that enqueues nothing;
 *   - inputs must be finite; NaN/Inf inputs give unspecified (but
 *     memory-safe) results;
 *   - outputs must not overlap inputs or each other (FP8W8A8_ERR_ALIAS);
 *   - faults inside a kernel surface at the caller's next synchronization.
 *
 * The library runs only on gfx950; any other current device gives
 * FP8W8A8_ERR_DEVICE.
 */
#ifndef FP8W8A8_H
#define FP8W8A8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fp8w8a8_status {
  FP8W8A8_OK = 0,
  FP8W8A8_ERR_NULL = 1,      /* a required pointer is NULL                  */
  FP8W8A8_ERR_SHAPE = 2,     /* a size or stride breaks the rules below     */
  FP8W8A8_ERR_ALIGN = 3,     /* a pointer is not 16-byte aligned            */
  FP8W8A8_ERR_ALIAS = 4,     /* an output overlaps an input or an output    */
  FP8W8A8_ERR_WORKSPACE = 5, /* workspace missing or smaller than required  */
  FP8W8A8_ERR_DEVICE = 6,    /* no HIP device, or the device is not gfx950  */
  FP8W8A8_ERR_HIP = 7        /* a HIP runtime call or kernel launch failed  */
} fp8w8a8_status;

/*
 * Channel-wise static weight quantization (the offline, one-shot step of the
 * FP8-Dynamic recipe; README "FP8-Dynamic": weights float8_e4m3fn,
 * channel-wise static).
 *   w        bf16 [n, k], row stride ldw >= k, ldw % 8 == 0 (input)
 *   qw       E4M3 [n, k], contiguous (row stride k)            (output)
 *   w_scale  float32 [n], one scale per output channel         (output)
 * Rules: n >= 0, k >= 1, k % 8 == 0; w, qw 16-byte aligned; w_scale 4-byte
 * aligned.  The result is bit-identical to the per-row definition above.
 */
int fp8w8a8_quantize_weight_channelwise(const uint16_t* w, int64_t n,
                                        int64_t k, int64_t ldw, uint8_t* qw,
                                        float* w_scale, void* stream);

/*
 * Per-token dynamic activation quantization (README "FP8-Dynamic": the input
 * activations of the quantized kernels are FP8, per token, dynamic).
 *   x        bf16 [m, k], row stride ldx >= k, ldx % 8 == 0   (input)
 *   qx       E4M3 [m, k], contiguous                           (output)
 *   x_scale  float32 [m]                                       (output)
 * Rules: m >= 0, k >= 1, k % 8 == 0; x, qx 16-byte aligned.
 */
int fp8w8a8_quantize_act_per_token(const uint16_t* x, int64_t m, int64_t k,
                                   int64_t ldx, uint8_t* qx, float* x_scale,
                                   void* stream);

/*
 * BF16 RMSNorm fused with the per-token quantization of its output: the norm
 * that precedes the q/k/v and gate/up Linears stays BF16 while those Linears
 * are FP8_DYNAMIC (MOSS-VL-Realtime-FP8 article, component / precision map),
 * and the norm's output row is the row whose amax the per-token scale needs.
 *   x        bf16 [m, k], row stride ldx >= k, ldx % 8 == 0     (input)
 *   gamma    bf16 [k], the norm weight                          (input)
 *   eps      float32, finite, >= 0                              (input)
 *   qx       E4M3 [m, k], contiguous                            (output)
 *   x_scale  float32 [m]                                        (output)
 *   y        bf16 [m, k], row stride ldy >= k, ldy % 8 == 0, the norm's
 *            output, or NULL to skip storing it (ldy then ignored) (output)
 * Per row (readings where the pages give no formula):
 *   t = bf16( x / sqrt(mean_k(x^2) + eps) )     evaluated in float32 with a
 *       power-of-two prescaling of the row (no overflow or underflow for
 *       any finite bf16 row) and a float64 square root, so t may differ by
 *       one bf16 step from the exactly rounded value where the exact value
 *       lies within float32 rounding error of a bf16 rounding boundary;
 *   y = bf16( gamma * t )                        (rounded once, exactly);
 *   qx, x_scale = the per-token quantization of y, bit-identical to
 *       fp8w8a8_quantize_act_per_token applied to y.
 * qx and x_scale feed fp8w8a8_fp8_linear directly.
 * Rules: m >= 0, k >= 8, k % 8 == 0; x, gamma, qx, y 16-byte aligned,
 * x_scale 4-byte aligned; gamma * t must stay finite.  Outputs must not
 * overlap the inputs or each other.
 */
int fp8w8a8_rmsnorm_quantize(const uint16_t* x, int64_t m, int64_t k,
                             int64_t ldx, const uint16_t* gamma, float eps,
                             uint8_t* qx, float* x_scale, uint16_t* y,
                             int64_t ldy, void* stream);

/*
 * The MLP activation fused with the per-token quantization of its output,
 * the input of down_proj.  gate_proj/up_proj (packed as gate_up_proj) and
 * down_proj are FP8_DYNAMIC Linears (MOSS-VL quantization README,
 * "FP8-Dynamic" and its packed-module mapping); the activation between
 * them stays BF16 (MOSS-VL-Realtime-FP8 article, component / precision map).
 *   gate     bf16 [m, n], row stride ldg >= n, ldg % 8 == 0       (input)
 *   up       bf16 [m, n], row stride ldu >= n, ldu % 8 == 0       (input)
 *            (for gate_up_proj's output Y [m, 2n]: gate = Y, up = Y + n,
 *            ldg = ldu = 2n)
 *   qh       E4M3 [m, n], contiguous                               (output)
 *   h_scale  float32 [m]                                           (output)
 *   h        bf16 [m, n], row stride ldh >= n, ldh % 8 == 0, the
 *            activation itself, or NULL to skip storing it       (output)
 * Per element (the pages do not name the activation; the gated SiLU is the
 * reading):
 *   s = bf16(silu(g)), silu(g) = g / (1 + exp(-g)), evaluated in float32
 *       (relative error below 2^-16 for every finite g whose result is a
 *       normal float), so s may differ by one bf16 step from the exactly
 *       rounded value where the exact value lies that close to a bf16
 *       rounding boundary;
 *   h = bf16(s * u)                              (rounded once, exactly);
 *   qh, h_scale = the per-token quantization of h, bit-identical to
 *       fp8w8a8_quantize_act_per_token applied to h.
 * Rules: m >= 0, n >= 8, n % 8 == 0; gate, up, qh, h 16-byte aligned,
 * h_scale 4-byte aligned; outputs must not overlap the inputs or each other.
 */
int fp8w8a8_swiglu_quantize(const uint16_t* gate, int64_t ldg,
                            const uint16_t* up, int64_t ldu, int64_t m,
                            int64_t n, uint8_t* qh, float* h_scale,
                            uint16_t* h, int64_t ldh, void* stream);

/*
 * FP8 E4M3 key/value-cache codec.  With the FP8 checkpoint under SGLang the
 * KV cache uses the engine's own dtype, e.g. --kv-cache-dtype fp8_e4m3
 * (MOSS-VL quantization README, "KV cache"); the pages give only the dtype.
 * Readings: each token's K (or V) row of `width` values (kv_heads x
 * head_dim) is quantized in groups of `group` consecutive values, each group
 * with one dynamic float32 scale = amax / 448 and codes exactly as
 * fp8w8a8_quantize_act_per_token would give for that group as a row; reading
 * back gives bf16(fl32(dec(code) * scale)).
 *
 * fp8w8a8_kv_quantize_fp8 (appending rows to a cache):
 *   kv       bf16 [rows, width], row stride ld >= width, ld % 8 == 0 (input)
 *   codes    E4M3 [rows, width], contiguous                          (output)
 *   scales   float32 [rows, width / group], contiguous               (output)
 * fp8w8a8_kv_dequantize_fp8 (reading a cache window back):
 *   codes, scales as above                                           (input)
 *   out      bf16 [rows, width], row stride ldo >= width, ldo % 8 == 0 (output)
 * Rules: rows >= 0; width >= 8, width % 8 == 0; group a power of two from 8
 * to 512 with width % group == 0; kv and out 16-byte aligned, codes 8-byte
 * aligned, scales 4-byte aligned; outputs must not overlap the inputs or
 * each other.  (To write rows t0.. of a cache, pass codes + t0 * width and
 * scales + t0 * width / group.)
 */
int fp8w8a8_kv_quantize_fp8(const uint16_t* kv, int64_t rows, int64_t width,
                            int64_t ld, int64_t group, uint8_t* codes,
                            float* scales, void* stream);
int fp8w8a8_kv_dequantize_fp8(const uint8_t* codes, const float* scales,
                              int64_t rows, int64_t width, int64_t group,
                              uint16_t* out, int64_t ldo, void* stream);

/*
 * INT8 group-wise key/value cache with a BF16 residual window.  The
 * checkpoint's Transformers path keeps the KV cache as HQQ INT8 with groups
 * of 64 and the newest 128 positions in BF16; reading it dequantizes the
 * history and appends that tail (MOSS-VL quantization README, "KV cache";
 * MOSS-VL-Realtime-FP8 article, KV-cache section).  HQQ's solver is not on
 * the pages; the reading is its asymmetric min-max starting point, each step
 * one IEEE float32 operation:
 *   per group:  s = fl32(fl32(max - min) / 255), stored with min (a zero
 *               max or min is taken as +0: the codes keep no sign of zero)
 *               q = clamp(rne(fl32(fl32(x - min) / s)), 0, 255)  (0 if s == 0)
 *   read back:  bf16(fl32(fl32(q * s) + min))
 * The caller keeps the newest tokens (up to the residual length, 128) as
 * bf16 and moves older ones into the INT8 store with
 * fp8w8a8_kv_quantize_int8 (at codes + t0 * width, scales / mins +
 * t0 * width / group).
 *
 * fp8w8a8_kv_quantize_int8:
 *   kv       bf16 [rows, width], row stride ld >= width, ld % 8 == 0 (input)
 *   codes    uint8 [rows, width], contiguous                         (output)
 *   scales, mins  float32 [rows, width / group], contiguous          (output)
 * fp8w8a8_kv_read_int8 (the cache read: history, then tail):
 *   codes, scales, mins  the INT8 store, hist rows                   (input)
 *   tail     bf16 [tail_rows, width], row stride ldt >= width, ldt % 8 == 0;
 *            may be NULL when tail_rows == 0                         (input)
 *   out      bf16 [hist + tail_rows, width], row stride ldo          (output)
 * Rules as for the FP8 codec (group a power of two from 8 to 512 dividing
 * width; the pages' group is 64); codes/scales/mins may be NULL when
 * hist == 0; tail 16-byte aligned.  A group whose max - min overflows
 * float32 (values beyond about +-1.7e38) gives unspecified codes.
 */
int fp8w8a8_kv_quantize_int8(const uint16_t* kv, int64_t rows, int64_t width,
                             int64_t ld, int64_t group, uint8_t* codes,
                             float* scales, float* mins, void* stream);
int fp8w8a8_kv_read_int8(const uint8_t* codes, const float* scales,
                         const float* mins, int64_t hist,
                         const uint16_t* tail, int64_t tail_rows, int64_t ldt,
                         int64_t width, int64_t group, uint16_t* out,
                         int64_t ldo, void* stream);

/*
 * The W8A8 Linear on already-quantized operands ("the quantized kernels" of
 * README "FP8-Dynamic"):
 *   y[m,n] = bf16_rne( (sum_k dec(qx[m,k]) * dec(qw[n,k])) * x_scale[m]
 *                      * w_scale[n] )
 * with float32 accumulation (summation order unspecified).
 *   qx, x_scale  from fp8w8a8_quantize_act_per_token, [m, k] and [m]
 *   qw, w_scale  from fp8w8a8_quantize_weight_channelwise, [n, k] and [n]
 *   y            bf16 [m, n], row stride ldy >= n, ldy % 8 == 0 (output)
 *   workspace    device scratch of at least
 *                fp8w8a8_workspace_bytes(m, n, k, 0) bytes; see below
 * Rules: m, n >= 0; n % 16 == 0; 128 <= k <= 4194304, k % 128 == 0; all
 * pointers 16-byte aligned.
 */
int fp8w8a8_fp8_linear(const uint8_t* qx, const float* x_scale,
                       const uint8_t* qw, const float* w_scale, int64_t m,
                       int64_t n, int64_t k, uint16_t* y, int64_t ldy,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * The same Linear with its output also quantized per token for the Linear
 * that reads it next (the dynamic per-token activation quantization of
 * README "FP8-Dynamic", applied to a layer's output where it is the next
 * layer's input): y exactly as fp8w8a8_fp8_linear gives it, and qy, y_scale
 * exactly as fp8w8a8_quantize_act_per_token(y) gives them.
 *   qx, x_scale, qw, w_scale, y, ldy, workspace  as for fp8w8a8_fp8_linear
 *                (the same workspace size)
 *   qy           uint8 [m, n] E4M3 codes of y, contiguous          (output)
 *   y_scale      float32 [m], amax of y's row / 448                (output)
 * Where the matmul splits K (a few hundred tokens or less on the tiled
 * GEMM) and n <= 16384, one kernel adds the splits, writes y and quantizes
 * it; otherwise the Linear's kernel, then the quantizer on y.
 * Rules as for fp8w8a8_fp8_linear; qy 16-byte and y_scale 4-byte aligned;
 * y, qy and y_scale overlap neither one another, nor an input, nor the
 * workspace.  Errors are returned before anything is launched.
 */
int fp8w8a8_fp8_linear_requant(const uint8_t* qx, const float* x_scale,
                               const uint8_t* qw, const float* w_scale, int64_t m,
                               int64_t n, int64_t k, uint16_t* y, int64_t ldy,
                               uint8_t* qy, float* y_scale, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * Fused FP8_DYNAMIC forward, bf16 in -> bf16 out: per-token quantization of
 * x (exactly as fp8w8a8_quantize_act_per_token) followed by
 * fp8w8a8_fp8_linear.  This is what a quantized Linear's forward is to its
 * caller.
 *   x        bf16 [m, k], row stride ldx >= k, ldx % 8 == 0   (input)
 *   qw, w_scale, y, ldy as for fp8w8a8_fp8_linear
 *   workspace    at least fp8w8a8_workspace_bytes(m, n, k, 1) bytes
 * Rules as for fp8w8a8_fp8_linear.
 */
int fp8w8a8_quant_linear(const uint16_t* x, int64_t ldx, const uint8_t* qw,
                         const float* w_scale, int64_t m, int64_t n, int64_t k,
                         uint16_t* y, int64_t ldy, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * The fused forward above for callers that cannot allocate or pass a
 * workspace: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same kernels and bit-identical results as
 * fp8w8a8_quant_linear; where that call would stage the quantized
 * activations (and float32 split-K partial sums) in the caller's
 * workspace, this one uses a device array of FP8W8A8_NOALLOC_SCRATCH_BYTES
 * bytes that the library holds on each GPU it runs on (from when the
 * library's code is loaded on that GPU until the process ends).  It calls
 * no allocating routine.
 *   x, ldx, qw, w_scale, m, n, k, y, ldy  as for fp8w8a8_quant_linear
 * Errors as for fp8w8a8_quant_linear, and FP8W8A8_ERR_WORKSPACE (nothing
 * launched) when the call needs more scratch than the array holds, i.e.
 * when fp8w8a8_workspace_bytes(m, n, k, 1) > FP8W8A8_NOALLOC_SCRATCH_BYTES
 * (roughly m * k > 64 Mi codes).  Decode-sized calls need no scratch.
 * All calls on one GPU share that GPU's array and it keeps the last call's
 * contents (nothing in it needs to start at zero): calls that may overlap
 * on one GPU (other streams, other threads) race, and the caller must
 * serialize them.
 */
#define FP8W8A8_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)
int fp8w8a8_quant_linear_noalloc(const uint16_t* x, int64_t ldx,
                                 const uint8_t* qw, const float* w_scale,
                                 int64_t m, int64_t n, int64_t k, uint16_t* y,
                                 int64_t ldy, void* stream);

/*
 * Several one-token FP8_DYNAMIC forwards in one launch: count independent
 * Linears at M = 1 (a decode step's projections: the README's
 * "FP8-Dynamic" Linears, whose decode speed is set by the weight bytes per
 * the MOSS-VL-Realtime-FP8 article, "why quantize"), each exactly
 * fp8w8a8_quant_linear(x, qw, w_scale) on one token, with bit-identical
 * output; one launch streams all their weights with one ramp-up and one
 * tail instead of one per Linear.
 *   items[i].x        bf16 [1, k] (one token), 16-byte aligned      (input)
 *   items[i].qw       E4M3 [n, k] contiguous, w_scale float32 [n]    (input)
 *   items[i].y        bf16 [1, n], 16-byte aligned                  (output)
 *   items[i].n, .k    n >= 16, n % 16 == 0, n < 2^31;
 *                     128 <= k <= 12288, k % 128 == 0
 * Rules: 1 <= count <= 16; items is a HOST array (read during the call
 * only); every y must overlap no input of any item and no other y.  No
 * workspace.  Errors are returned before anything is launched.
 */
typedef struct fp8w8a8_group_linear {
  const uint16_t* x;
  const uint8_t* qw;
  const float* w_scale;
  uint16_t* y;
  int64_t n;
  int64_t k;
} fp8w8a8_group_linear;
int fp8w8a8_quant_linear_group_m1(const fp8w8a8_group_linear* items, int count,
                                  void* stream);

/*
 * Per-token dynamic quantization of several activation matrices in one
 * launch: count independent fp8w8a8_quantize_act_per_token calls (README
 * "FP8-Dynamic": activations FP8 per token, dynamic), each item's codes and
 * scales bit-identical to that call -- e.g. the inputs of a decode step's
 * Linears ahead of one fp8w8a8_fp8_linear_group.
 *   items[i].x        bf16 [m, k], row stride ldx >= k, ldx % 8 == 0  (input)
 *   items[i].qx       E4M3 [m, k], contiguous                         (output)
 *   items[i].x_scale  float32 [m]                                     (output)
 * Rules: 1 <= count <= 16; items is a HOST array (read during the call
 * only); per item m >= 0, 8 <= k <= 16384, k % 8 == 0, x and qx 16-byte
 * aligned, x_scale 4-byte aligned; no output may overlap any item's input
 * or another output.  An item with m == 0 is skipped (its pointers may be
 * NULL).  Errors are returned before anything is launched.
 */
typedef struct fp8w8a8_group_quant {
  const uint16_t* x;
  int64_t m;
  int64_t k;
  int64_t ldx;
  uint8_t* qx;
  float* x_scale;
} fp8w8a8_group_quant;
int fp8w8a8_quantize_act_group(const fp8w8a8_group_quant* items, int count,
                               void* stream);

/*
 * E4M3 weight codes in MFMA-tile order, the weight layout of
 * fp8w8a8_fp8_linear_group.  An offline step next to the channel-wise
 * quantization (README "FP8-Dynamic": the weights are quantized once,
 * statically); a pure byte permutation, its codes and scales unchanged.
 *   qw      E4M3 [n, k], contiguous (row-major, as quantized)     (input)
 *   tiled   n * k bytes                                          (output)
 * Layout: K in panels of four 128-byte K blocks (the last panel holds the
 * ipp(p) = min(4, k / 128 - 4 p) blocks left); for panel p, row block rb
 * (16 rows), block j of the panel (K block i = 4 p + j), h in {0, 1},
 * l in [0, 64), e in [0, 16):
 *   tiled[p * n * 512 + (rb * ipp(p) + j) * 2048 + h * 1024 + 16 * l + e]
 *     = qw[16 * rb + (l % 16), 128 * i + 64 * h + 16 * (l / 16) + e]
 * i.e. each 16 x 128-byte block is one contiguous 2 KB tile, a panel holds
 * the tiles of every row block for its 512 bytes of K (row block by row
 * block), and the panels follow each other in K order.
 * Rules: n >= 0, n % 16 == 0; 128 <= k <= 16384, k % 128 == 0; both pointers
 * 16-byte aligned; the two ranges must not overlap.
 */
int fp8w8a8_tile_weights(const uint8_t* qw, int64_t n, int64_t k, uint8_t* tiled,
                         void* stream);

/*
 * Several Linears on already-quantized operands at a few tokens, in one
 * launch: count independent fp8w8a8_fp8_linear calls (README "FP8-Dynamic":
 * per-token dynamic E4M3 activations, channel-wise E4M3 weights) at one
 * token count m, each
 *   y[m,n] = bf16_rne( (sum_k dec(qx[m,k]) * dec(qw[n,k])) * x_scale[m]
 *                      * w_scale[n] )
 * with float32 accumulation (summation order unspecified; each output is
 * one thread's sum over K in ascending order of 128-byte blocks, the same
 * whatever the grouping).  At a few tokens the Linears are bound by their
 * weight bytes (MOSS-VL-Realtime-FP8 article, "why quantize"); one launch
 * streams every item's weights with one ramp-up and one tail, and items may
 * share their codes (e.g. the Linears of a layer that read the same input,
 * quantized once).
 *   items[i].qx       E4M3 [m, k] contiguous, x_scale float32 [m]     (input)
 *   items[i].qw_tiled the item's [n, k] weight codes in the order of
 *                     fp8w8a8_tile_weights, w_scale float32 [n]      (input)
 *   items[i].y        bf16 [m, n] contiguous                         (output)
 *   items[i].n, .k    64 <= n <= 2^24, n % 64 == 0, m * n <= 2^30;
 *                     128 <= k <= 16384, k % 128 == 0
 * Rules: 1 <= m <= 256; 1 <= count <= 16; items is a HOST array (read during
 * the call only); all pointers 16-byte aligned; every y must overlap no
 * input of any item and no other y.  No workspace.  Errors are returned
 * before anything is launched.
 */
typedef struct fp8w8a8_group_fp8_linear {
  const uint8_t* qx;
  const float* x_scale;
  const uint8_t* qw_tiled;
  const float* w_scale;
  uint16_t* y;
  int64_t n;
  int64_t k;
} fp8w8a8_group_fp8_linear;
int fp8w8a8_fp8_linear_group(const fp8w8a8_group_fp8_linear* items, int count,
                             int64_t m, void* stream);

/*
 * fp8w8a8_fp8_linear_group with one item, items[rq], summed over K in
 * several ranges, and optionally its output also quantized per token for
 * the Linear that reads it next (README "FP8-Dynamic": dynamic per-token
 * activation scales, here for a layer's output that is the next layer's
 * input, as fp8w8a8_fp8_linear_requant does for one Linear).  At a few
 * tokens a long-K Linear (e.g. down, K = 12288) has few 64-row units, each
 * three times as long as those of the K = 4096 Linears, and becomes the
 * launch's long pole or leaves the GPU half idle (MOSS-VL-Realtime-FP8
 * article, "why quantize": these Linears are bound by their weight bytes);
 * here its K is summed in several ranges, each range its own units of the
 * one launch beside the other items, and one more kernel adds the ranges
 * in order, writes y and, if asked, quantizes it:
 *   items[rq].y   exactly what the raw float32 sum of the ranges, added in
 *                 range order, gives through the epilogue
 *                 bf16_rne(sum * x_scale[m] * w_scale[n]) (summation order
 *                 unspecified, so within the tolerance of any float32 sum)
 *   qy            uint8 [m, items[rq].n] E4M3 codes of that y, contiguous,
 *                 and y_scale float32 [m]: exactly
 *                 fp8w8a8_quantize_act_per_token(y); both NULL: y only
 *                 (output)
 *   every other item exactly as fp8w8a8_fp8_linear_group gives it
 *   workspace     device scratch of at least
 *                 fp8w8a8_group_requant_workspace_bytes(items, count, m, rq)
 *                 bytes (float32 sums [ranges, m, n]; no state survives a
 *                 call; calls that may run concurrently need distinct ones)
 * Rules: those of fp8w8a8_fp8_linear_group; 0 <= rq < count; qy and
 * y_scale both given or both NULL; items[rq].n <= 2^20, and with them
 * items[rq].n <= 16384, qy
 * 16-byte and y_scale 4-byte aligned; the workspace 16-byte aligned; qy,
 * y_scale and the workspace overlap no input, no y and one another.  Errors
 * are returned before anything is launched.
 * fp8w8a8_group_requant_workspace_bytes returns 0 for invalid arguments.
 */
size_t fp8w8a8_group_requant_workspace_bytes(const fp8w8a8_group_fp8_linear* items,
                                             int count, int64_t m, int rq);
int fp8w8a8_fp8_linear_group_requant(const fp8w8a8_group_fp8_linear* items, int count,
                                     int64_t m, int rq, uint8_t* qy, float* y_scale,
                                     void* workspace, size_t workspace_bytes,
                                     void* stream);

/*
 * The adjacent fusions followed by the Linear, in one call: exactly
 * fp8w8a8_rmsnorm_quantize(x, gamma, eps) (or fp8w8a8_swiglu_quantize(gate,
 * up)) followed by fp8w8a8_fp8_linear, with bit-identical output.  The norm
 * ahead of q/k/v and gate/up and the activation ahead of down stay BF16
 * while the Linears after them are FP8_DYNAMIC (MOSS-VL-Realtime-FP8
 * article, component / precision map; MOSS-VL quantization README,
 * "FP8-Dynamic").  At decode
 * sizes (2 <= m <= 4 and m * k <= 16384, or m == 1 and k > 4096; for the
 * norm also k % 512 == 0) the norm or activation runs inside the decode
 * GEMV's activation staging, one kernel in all; otherwise (including one
 * token with k <= 4096, where two kernels are faster) its codes go through
 * the workspace.
 *   x / gate bf16 [m, k], row stride ldx / ldg >= k, % 8 == 0        (input)
 *   gamma    bf16 [k]                                                (input)
 *   up       bf16 [m, k], row stride ldu >= k, ldu % 8 == 0          (input)
 *   qw, w_scale, y, ldy as for fp8w8a8_fp8_linear
 *   workspace    at least fp8w8a8_workspace_bytes(m, n, k, 2) (norm) or
 *                (m, n, k, 3) (activation) bytes
 * Rules as for fp8w8a8_fp8_linear and for the two fused steps (eps finite
 * and >= 0; y may overlap none of the inputs, nor the workspace); errors
 * are returned before anything is launched.
 */
int fp8w8a8_rmsnorm_quant_linear(const uint16_t* x, int64_t ldx,
                                 const uint16_t* gamma, float eps,
                                 const uint8_t* qw, const float* w_scale,
                                 int64_t m, int64_t n, int64_t k, uint16_t* y,
                                 int64_t ldy, void* workspace,
                                 size_t workspace_bytes, void* stream);
int fp8w8a8_swiglu_quant_linear(const uint16_t* gate, int64_t ldg,
                                const uint16_t* up, int64_t ldu,
                                const uint8_t* qw, const float* w_scale,
                                int64_t m, int64_t n, int64_t k, uint16_t* y,
                                int64_t ldy, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * Workspace size in bytes for fp8w8a8_fp8_linear (fused == 0),
 * fp8w8a8_quant_linear (fused == 1, or any value other than 0, 2, 3),
 * fp8w8a8_rmsnorm_quant_linear (fused == 2) or
 * fp8w8a8_swiglu_quant_linear (fused == 3) at the given sizes; 0 when the call needs
 * none, and 0 for invalid sizes.  The workspace is plain scratch that holds
 * the quantized activations [m, k] and their scales [m] when a fused call
 * quantizes in a separate kernel before the matmul, and float32 partial sums
 * [splits, m, n] when the matmul splits K over several workgroups (shapes
 * with few output tiles, i.e. m from 17 to a few hundred; the splits are
 * added in a fixed order, so results are deterministic); no state survives
 * a call, so any workspace can be reused, but calls that may run
 * concurrently need distinct workspaces.
 */
size_t fp8w8a8_workspace_bytes(int64_t m, int64_t n, int64_t k, int fused);

/*
 * Zero-fill a device buffer (e.g. a workspace) with a kernel on `stream`
 * (no hipMemsetAsync, so it can sit inside a captured graph).
 * bytes % 16 == 0, buffer 16-byte aligned.
 */
int fp8w8a8_workspace_init(void* workspace, size_t bytes, void* stream);

/* Human-readable name of a status code (static string, never NULL). */
const char* fp8w8a8_status_string(int status);

/* The hipError_t behind the calling thread's last FP8W8A8_ERR_HIP or
 * FP8W8A8_ERR_DEVICE (0 if none). */
int fp8w8a8_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8W8A8_H */
