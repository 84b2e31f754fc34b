/*
 * strata_moe.h - C ABI of a routed mixture-of-experts FFN layer for AMD
 * Instinct MI355X (gfx950).
 *
 * The layer, as the Strata pages describe it:
 *   - each layer's router selects a few experts out of a large pool for every
 *     token (512 experts, about 10 active): "两天移植，预填充提速8倍：Strata
 *     引擎实测" (kongchang.com), section "Strata快在哪：不是魔法，是物流", MoE
 *     note; penglei.dev "Strata local MoE", section "原理一";
 *   - tokens routed to the same expert are processed as one batch so that the
 *     expert's weights are fetched once for all of them (same kongchang.com
 *     section: bigger prefill batches reuse each expert over more tokens);
 *   - expert matmuls run on group-quantized 4-bit weights, dequantized inside
 *     the matmul kernel rather than into a full-precision copy first
 *     (lqnn.cn static review, §1.2 and §3.1; kongchang.com, MMQ note);
 *   - the expert FFN is SwiGLU, down(silu(gate x) * up x), and the selected
 *     experts' outputs are summed with softmax routing weights.
 *
 * Conventions shared by every call:
 *   - Every array pointer is a DEVICE pointer owned by the caller; the library
 *     keeps no reference after the call returns.  Arrays must be 16-byte
 *     aligned; workspaces 256-byte aligned.
 *   - `stream` is a hipStream_t passed as void* (NULL: the null stream).
 *     Calls only enqueue work on `stream`: they never synchronize, never
 *     allocate device memory and never read device data back to the host.
 *   - Arguments are checked before anything is enqueued.  A failed check
 *     returns a non-zero strata_status and enqueues nothing;
 *     strata_moe_last_error() then names the parameter and its value
 *     (explicit errors, no silent fallback to another path: yfxerp.com
 *     static review, §5.2 and §6.2).  A HIP launch failure returns
 *     STRATA_ERR_HIP with the HIP error string appended.
 *   - T == 0 is valid and enqueues nothing, except that strata_moe_permute
 *     still writes counts[] = 0 and offsets[] = 0.
 *   - Logits must be finite; non-finite logits give unspecified routing.
 *
 * Supported envelope (outside it: STRATA_ERR_UNSUPPORTED):
 *   1 <= E <= 1024, 1 <= k <= min(E, 32) (k > E: STRATA_ERR_INVALID_ARGUMENT),
 *   T*k < 2^31, g in {32, 64, 128}, H % 256 == 0, I % 128 == 0,
 *   256 <= H <= 16384, 128 <= I <= 16384.
 */
#ifndef STRATA_MOE_H
#define STRATA_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  STRATA_OK = 0,
  STRATA_ERR_INVALID_ARGUMENT = 1, /* null pointer, negative size, k > E, misalignment */
  STRATA_ERR_UNSUPPORTED = 2,      /* a size outside the supported envelope */
  STRATA_ERR_WORKSPACE = 3,        /* workspace missing or smaller than required */
  STRATA_ERR_HIP = 4               /* the HIP runtime reported an error */
} strata_status;

/*
 * Weight formats of strata_moe_weights.format.
 *   STRATA_W_INT4       symmetric 4-bit codes, q = u - 8.
 *   STRATA_W_INT4_ASYM  asymmetric 4-bit: each group stores a scale and a zero
 *                       point z in [0, 15], q = u - z (lqnn.cn static review,
 *                       §3.1: per-group scale and zero point).
 *   STRATA_W_INT5       symmetric 5-bit blocks, q = u + 16 b - 16 in [-16, 15]
 *                       with a fifth bit b per element (4- and 5-bit block
 *                       quantization: kongchang.com hands-on, section
 *                       "Strata快在哪：不是魔法，是物流", MMQ note).
 */
typedef enum {
  STRATA_W_INT4 = 0,
  STRATA_W_INT4_ASYM = 1,
  STRATA_W_INT5 = 2
} strata_weight_format;

/*
 * Byte layouts of the packed codes (gate, up, down) of strata_moe_weights.
 *   STRATA_L_ROWS   row-major: byte j of row n of expert e at
 *                   (e*N + n) * K/2 + j.
 *   STRATA_L_TILED  32-row x 64-byte tiles: with r = e*N + n,
 *                   byte ((r/32) * (K/128) + j/64) * 2048 + (r%32) * 64 + j%64.
 *                   Every 128-wide K stage of 32 rows is one contiguous
 *                   2 KB run, so the grouped matrix-core GEMMs, which stream
 *                   a stage of many rows at a time, read whole cache lines
 *                   (the row-major layout gives them half lines and about
 *                   twice the fetched bytes).  Every call that takes weights
 *                   reads both layouts with the same results, bit for bit;
 *                   strata_moe_tile_weights converts once at load time.
 * Scales, zero points and fifth-bit words are row-major in both.
 */
typedef enum {
  STRATA_L_ROWS = 0,
  STRATA_L_TILED = 1
} strata_weight_layout;

/*
 * Group-quantized expert weights (all device pointers, caller-owned).
 *
 * Each matrix W[N][K] (gate, up: N = I, K = H; down: N = H, K = I) holds
 * codes q, K-contiguous rows, one nibble u (the code's low 4 bits, offset
 * binary) per element and two per byte: byte j of a row = u(2j) | u(2j+1) << 4
 * (even K index in the low nibble).  One IEEE fp16 scale per g consecutive K
 * elements: W[n][kk] = q[n][kk] * scale[n][kk / g], where q follows `format`:
 *   STRATA_W_INT4       q = u - 8.  gate_zero .. down_hi must be NULL.
 *   STRATA_W_INT4_ASYM  q = u - z[n][kk / g]; the zero points of a row are
 *                       packed two per byte (group j in byte j / 2, even j in
 *                       the low nibble): gate_zero, up_zero [E][I][H/g/2],
 *                       down_zero [E][H][I/g/2].  H/g and I/g must be even.
 *   STRATA_W_INT5       q = u + 16 b - 16; the fifth bit b of element
 *                       kk = 32m + 8c + i (c in 0..3, i in 0..7) is bit
 *                       4i + c of the 32-bit word hi[n][m]: gate_hi, up_hi
 *                       [E][I][H/32], down_hi [E][H][I/32] (4-byte aligned).
 * (Grouped 4-bit weights with per-group scales: lqnn.cn static review §3.1,
 * group sizes 32/64/128; yfxerp.com static review §3.1.)
 */
typedef struct {
  const uint8_t *gate;        /* [E][I][H/2] */
  const uint16_t *gate_scale; /* fp16 bits, [E][I][H/g] */
  const uint8_t *up;          /* [E][I][H/2] */
  const uint16_t *up_scale;   /* fp16 bits, [E][I][H/g] */
  const uint8_t *down;        /* [E][H][I/2] */
  const uint16_t *down_scale; /* fp16 bits, [E][H][I/g] */
  int32_t num_experts;        /* E */
  int32_t hidden;             /* H */
  int32_t inter;              /* I */
  int32_t group;              /* g */
  int32_t format;             /* strata_weight_format; 0 (zero-initialised) = STRATA_W_INT4 */
  const uint8_t *gate_zero;   /* STRATA_W_INT4_ASYM only, else NULL */
  const uint8_t *up_zero;
  const uint8_t *down_zero;
  const uint32_t *gate_hi;    /* STRATA_W_INT5 only, else NULL */
  const uint32_t *up_hi;
  const uint32_t *down_hi;
  int32_t layout;             /* strata_weight_layout of gate, up, down; 0 = STRATA_L_ROWS */
} strata_moe_weights;

/*
 * strata_moe_route - top-k expert selection with softmax gating.
 * (Router picks a few experts per token: kongchang.com hands-on, section
 * "Strata快在哪", MoE note; penglei.dev, "原理一".)
 *
 *   logits    in  float32 [T][E] router logits (row-major).
 *   topk_ids  out int32   [T][k] selected experts per token, by descending
 *                         logit; equal logits go to the lower expert index,
 *                         and -0.0 equals +0.0.  Bit-exact and deterministic.
 *   topk_w    out float32 [T][k] softmax over the k selected logits,
 *                         w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0).
 */
int strata_moe_route(const float *logits, int32_t T, int32_t E, int32_t k,
                     int32_t *topk_ids, float *topk_w, void *stream);

/*
 * strata_moe_router - the router projection in front of the top-k selection:
 * logits = x . W_r^T, then exactly strata_moe_route on those logits.  (The
 * router that scores the experts of each token before a few are picked:
 * "两天移植，预填充提速8倍：Strata引擎实测" (kongchang.com), section
 * "Strata快在哪：不是魔法，是物流", MoE note.)
 *
 *   x_bf16         in  bf16 bits [T][H], row-major.
 *   w_router_bf16  in  bf16 bits [E][H], row-major (one row per expert).
 *   logits         out float32 [T][E]: sum_h x[t][h] * W_r[e][h], products
 *                  exact in fp32, accumulated in fp32 (MFMA order).
 *   topk_ids, topk_w  out as from strata_moe_route on `logits`.
 *
 * H must be a multiple of 64 in [64, 16384], T*H and E*H below 2^30; E and
 * k as for strata_moe_route.  T = 0 does nothing.  Pointers 16-byte aligned.
 */
int strata_moe_router(const uint16_t *x_bf16, int32_t T, int32_t H, const uint16_t *w_router_bf16, int32_t E,
                      int32_t k, float *logits, int32_t *topk_ids, float *topk_w, void *stream);

/*
 * strata_moe_permute - group the T*k (token, slot) pairs by expert.
 * (Tokens routed to one expert are batched together: kongchang.com hands-on,
 * section "Strata快在哪".)
 *
 * Pair p = t*k + j refers to topk_ids[t][j].
 *   topk_ids  in  int32 [T*k], values in [0, E).
 *   counts    out int32 [E]    pairs routed to each expert.
 *   offsets   out int32 [E+1]  exclusive prefix sum of counts; offsets[E] = T*k.
 *   perm      out int32 [T*k]  perm[offsets[e] + r] = the r-th pair (ascending p)
 *                              routed to expert e.
 *   inv_perm  out int32 [T*k]  inv_perm[perm[i]] = i.
 *   workspace     device scratch of at least
 *                 strata_moe_permute_workspace_size(T, E, k) bytes (NULL
 *                 when that is 0).
 * All outputs are bit-exact and deterministic (no dependence on the order of
 * atomic operations).  Expert ids outside [0, E) are a precondition violation.
 */
int strata_moe_permute(const int32_t *topk_ids, int32_t T, int32_t E, int32_t k,
                       int32_t *counts, int32_t *offsets, int32_t *perm,
                       int32_t *inv_perm, void *workspace, size_t workspace_bytes,
                       void *stream);

/*
 * strata_moe_ffn - SwiGLU expert FFN over the grouped pairs, with the int4
 * dequantization fused into the expert matmul kernels.
 * (Dequantize inside the kernel, not before the matmul: lqnn.cn static
 * review §1.2; activation fused with the FFN projection: yfxerp.com static
 * review §5.1.)
 *
 *   x_bf16    in  bfloat16 bits [T][H] token activations.  The expert
 *                 matmuls run with fp16 operands and fp32 accumulation; see
 *                 "fp16 operand envelope" below.
 *   w         in  host pointer to the weight descriptor (device arrays).
 *   offsets   in  int32 [E+1] and perm int32 [T*k], as from strata_moe_permute.
 *   topk_w    in  float32 [T*k] routing weights, or NULL.
 *   y_or_out  out float32:
 *             topk_w != NULL: out[T][H] = sum_j topk_w[t][j] * y(t, j); the
 *                 library overwrites all of out.  The expert outputs pass
 *                 through fp16 rows in workspace (pair order) and a final
 *                 kernel sums each token's k rows in j order in fp32, so the
 *                 result is deterministic;
 *             topk_w == NULL: y[T*k][H] in grouped order, row i = the expert
 *                 output of pair perm[i] (deterministic); finish the layer
 *                 with strata_moe_combine.
 *   workspace     device scratch, at least strata_moe_workspace_size() bytes.
 *
 * Path selection: a bandwidth-bound GEMV path streams each selected expert's
 * weights once for decode and draft-verify batches (T <= 16, hidden in
 * {256, 512, 1024, 2048, 4096}, inter a power of two in [128, 2048]);
 * otherwise grouped GEMMs on the matrix cores.  Environment variable
 * STRATA_MOE_FFN_PATH = auto (default) | gemm | gemv, read on every call,
 * forces one of them; forcing gemv outside its envelope returns
 * STRATA_ERR_UNSUPPORTED, any other value STRATA_ERR_INVALID_ARGUMENT.
 */
int strata_moe_ffn(const uint16_t *x_bf16, int32_t T, int32_t k,
                   const strata_moe_weights *w, const int32_t *offsets,
                   const int32_t *perm, const float *topk_w, float *y_or_out,
                   void *workspace, size_t workspace_bytes, void *stream);

/*
 * fp16 operand envelope (strata_moe_ffn and strata_moe_layer).  The matrix
 * and dot-product units take fp16 operands (the same matrix-core rate as
 * bf16, with 3 more mantissa bits); accumulation is fp32.  Three values pass
 * through fp16:
 *   x   each bf16 activation is converted with round-toward-zero: exact for
 *       2^-14 <= |x| <= 65504; |x| < 2^-14 becomes an fp16 subnormal
 *       (absolute error < 2^-24); |x| > 65504 saturates to +-65504.
 *   h   silu(gate . x) * (up . x) per pair and intermediate column, rounded
 *       to nearest fp16: |h| must stay <= 65504 (beyond it h becomes +-inf
 *       and the output is unspecified); |h| < 2^-14 is kept as a subnormal
 *       (absolute error <= 2^-25; on the decode paths every other pair of
 *       columns is held divided by 16, so there the subnormal range starts
 *       at |h| < 2^-10).
 *   y   each pair's expert output W_down . h, in fused mode on the grouped-
 *       GEMM and GEMV paths, rounded to nearest fp16 before the weighted
 *       sum: |y| must stay <= 65504.  The unfused mode writes y in fp32, and
 *       the two-kernel decode layer never rounds y.
 * Inside this envelope the output meets max |err| <= 2e-2 * RMS(out) and
 * sum |err| / sum |out| <= 5e-3 against an exact evaluation; activations far
 * below 2^-14 throughout a token lose relative accuracy to the subnormals.
 */

/*
 * strata_moe_combine - weighted sum of each token's expert outputs, the last
 * step of the routed layer: the selected experts' outputs are added up with
 * the softmax routing weights of strata_moe_route (the layer as the
 * kongchang.com hands-on describes it, section "Strata快在哪：不是魔法，是
 * 物流", MoE note: each token's few active experts together form the layer's
 * output; the weighting is the softmax over the selected logits).
 *
 *   y         in  float32 [T*k][H] grouped-order expert outputs.
 *   inv_perm  in  int32 [T*k]; topk_w in float32 [T*k].
 *   out       out float32 [T][H], out[t] = sum_{j=0}^{k-1} topk_w[t*k+j] *
 *                 y[inv_perm[t*k+j]], summed in j order (deterministic).
 */
int strata_moe_combine(const float *y, const int32_t *inv_perm, const float *topk_w,
                       int32_t T, int32_t k, int32_t H, float *out, void *stream);

/*
 * strata_moe_layer - the whole routed FFN layer in one call: routing,
 * grouping, the expert FFN and the weighted combine, i.e. strata_moe_route,
 * strata_moe_permute and strata_moe_ffn (with topk_w) in order on one
 * workspace.  (The layer as a whole: "两天移植，预填充提速8倍：Strata引擎实测"
 * (kongchang.com), section "Strata快在哪：不是魔法，是物流".)
 *
 *   logits, x_bf16, T, k, w  in  as for strata_moe_route and strata_moe_ffn.
 *   topk_ids, topk_w         out as from strata_moe_route (bit-identical).
 *   counts, offsets, perm, inv_perm
 *                            out as from strata_moe_permute (bit-identical).
 *   out        out float32 [T][H], the layer output (overwritten).
 *   workspace  device scratch, at least strata_moe_workspace_size() bytes,
 *              256-byte aligned.
 *
 * Decode batches (T <= 16, k <= 16, k * inter <= 16384, hidden in {256, ...,
 * 4096}, inter a power of two in [128, 2048]; STRATA_MOE_FFN_PATH auto or
 * gemv) run as two kernels: every expert row block re-selects its token's
 * expert itself while dedicated blocks write the routing outputs, and the
 * down projection is token-major: out[t][n] = sum_j topk_w[t][j] *
 * (W_down[e_j][n] . h(t, j)) in fp32, summed in j order (deterministic, and
 * without the fp16 rounding of y that the three-call path stores).  Other
 * shapes, or STRATA_MOE_FFN_PATH=gemm, run the three calls' kernels; on the
 * grouped-GEMM path with more than 1024 pairs the routing kernel also
 * converts x for the GEMM and the grouping scan also builds the GEMM's tile
 * lists, so the ffn's prologue kernel is not launched (same results).
 * Argument errors are those of the three calls; T = 0 writes counts and
 * offsets (zeros) only.
 */
int strata_moe_layer(const float *logits, const uint16_t *x_bf16, int32_t T, int32_t k,
                     const strata_moe_weights *w, int32_t *topk_ids, float *topk_w,
                     int32_t *counts, int32_t *offsets, int32_t *perm, int32_t *inv_perm,
                     float *out, void *workspace, size_t workspace_bytes, void *stream);

/*
 * strata_moe_layer_noalloc - strata_moe_layer without a workspace argument,
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  It runs
 * the same kernels as strata_moe_layer (same results, bit for bit) on a
 * scratch array that the library holds in static device memory: one copy of
 * STRATA_MOE_NOALLOC_SCRATCH_BYTES per device the library runs on, kept until
 * the process ends.  The call allocates nothing; the caller still provides
 * every input and output array.
 *
 *   Arguments as for strata_moe_layer, without workspace / workspace_bytes.
 *   Shapes whose workspace (strata_moe_workspace_size) exceeds
 *   STRATA_MOE_NOALLOC_SCRATCH_BYTES return STRATA_ERR_UNSUPPORTED with the
 *   required and available bytes in the message (e.g. a decode batch or a
 *   512-token prefill at H = 2048, I = 512, E = 512, k = 10 fit; the
 *   6144-token chunk does not).
 *   All calls on one device share that device's scratch array: calls that
 *   overlap in time on one device (concurrent streams, several host threads)
 *   race on it and must be serialized by the caller.  The scratch keeps the
 *   last call's contents; no result depends on them.
 */
#define STRATA_MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int strata_moe_layer_noalloc(const float *logits, const uint16_t *x_bf16, int32_t T, int32_t k,
                             const strata_moe_weights *w, int32_t *topk_ids, float *topk_w, int32_t *counts,
                             int32_t *offsets, int32_t *perm, int32_t *inv_perm, float *out, void *stream);

/*
 * strata_moe_tile_weights - rewrite one packed-code array from STRATA_L_ROWS
 * to STRATA_L_TILED (a permutation of its bytes; see strata_weight_layout).
 * Call it once per matrix (gate, up, down) when the weights are loaded.
 *
 *   src   in  uint8 [rows][K/2], row-major packed codes; rows = E*N of the
 *             matrix (E*I for gate and up, E*H for down), K its row length.
 *   dst   out uint8, rows*K/2 bytes in the tiled layout.  Must not overlap
 *             src.  Both 16-byte aligned.
 *   rows  a multiple of 32, K a multiple of 128 (every matrix in the
 *         supported envelope qualifies); rows = 0 enqueues nothing.
 *         Otherwise STRATA_ERR_INVALID_ARGUMENT.
 */
int strata_moe_tile_weights(const uint8_t *src, uint8_t *dst, int64_t rows, int32_t K, void *stream);

/*
 * Bytes of device workspace that strata_moe_permute, strata_moe_ffn and
 * strata_moe_layer need for this shape (the ffn's regions plus the grouping
 * histogram's, which strata_moe_layer keeps apart).  Returns 0 for invalid
 * sizes.
 */
size_t strata_moe_workspace_size(int32_t T, int32_t E, int32_t k, int32_t H,
                                 int32_t I, int32_t g);

/*
 * Bytes of device workspace that strata_moe_permute alone needs for T tokens,
 * E experts and top-k (0 when no workspace is needed, e.g. at most 1024
 * pairs; (size_t)-1 for invalid sizes).  strata_moe_workspace_size covers it.
 */
size_t strata_moe_permute_workspace_size(int32_t T, int32_t E, int32_t k);

/*
 * 4-bit KV cache and sparse attention over it.
 *
 * The key/value cache can be stored in 4 bits per element (the optional
 * 4-bit KV cache of "40天64个版本：Strata如何用发版密度定义AI本地推理路线图",
 * release 0.1.8), quantized per head and symmetrically (lqnn.cn static
 * review, §3.1), with the dequantization fused into the operator that reads
 * the cache (yfxerp.com static review, §4.2).  The attention reads only the
 * ~2000 cache rows that an indexer selected for each query
 * ("两天移植，预填充提速8倍：Strata引擎实测" (kongchang.com), section
 * "Strata快在哪：不是魔法，是物流", attention paragraph).
 *
 * Cache format (one array for keys, one for values): codes uint8 [L][Hkv][D/2]
 * holding offset-binary nibbles u = q + 8 (even element in the low nibble)
 * and scales fp16 [L][Hkv], one per (position, head) vector:
 * x[l][h][d] = (u - 8) * scale[l][h].  Supported: D = 128, Hkv in {1, 2, 4, 8}
 * (outside: STRATA_ERR_UNSUPPORTED).
 */

/*
 * strata_kv_quantize - write T new (token, head) vectors into the cache.
 *
 *   x_bf16   in  bf16 bits [T][Hkv][D].
 *   slots    in  int32 [T]: cache position of token t; rows whose slot lies
 *                outside [0, L) are skipped.
 *   codes    out uint8 [L][Hkv][D/2], rows slots[t] written.
 *   scales   out fp16 bits [L][Hkv], rows slots[t] written.
 * Per vector: s = fp16(max|x| / 7) and q = clamp(rint(x / s), -8, 7), the
 * division and rounding in IEEE fp32 (nearest-even); an all-zero vector gets
 * s = 0 and codes 8.  Bit-exact and deterministic.  Inputs must satisfy
 * max|x| <= 7 * 65504 (beyond it the fp16 scale overflows to inf).  Two
 * tokens with the same slot race (the last write is unspecified).
 */
int strata_kv_quantize(const uint16_t *x_bf16, int32_t T, int32_t Hkv, int32_t D, const int32_t *slots,
                       uint8_t *codes, uint16_t *scales, int32_t L, void *stream);

/*
 * strata_kv_quantize_pair - strata_kv_quantize of the keys and the values of
 * the same T tokens in one launch (each token's K and V vectors are cached
 * together; one launch instead of two halves the fixed launch and memory-
 * latency cost, which dominates at decode sizes).
 *
 *   k_bf16, v_bf16   in  bf16 bits [T][Hkv][D] each.
 *   slots            in  int32 [T], shared by both (as in strata_kv_quantize).
 *   k_codes, k_scales, v_codes, v_scales  out  the key and the value cache
 *                    arrays ([L][Hkv][D/2] uint8, [L][Hkv] fp16 bits).
 * Every written byte equals what two strata_kv_quantize calls write (same
 * arithmetic, bit-exact); errors as there, T * Hkv * 2 < 2^31.
 */
int strata_kv_quantize_pair(const uint16_t *k_bf16, const uint16_t *v_bf16, int32_t T, int32_t Hkv, int32_t D,
                            const int32_t *slots, uint8_t *k_codes, uint16_t *k_scales, uint8_t *v_codes,
                            uint16_t *v_scales, int32_t L, void *stream);

/*
 * strata_sparse_attention - attention of Tq queries over selected positions
 * of a 4-bit cache, dequantizing the selected rows as they are read.
 *
 *   q_bf16   in  bf16 bits [Tq][Hq][D]; query head h reads KV head
 *                h / (Hq / Hkv) (Hq / Hkv in {1, 2, 4}).
 *   k_codes, k_scales, v_codes, v_scales  in  the cache, as above, L positions.
 *   sel      in  int32 [Tq][n_sel] cache positions per query (each in
 *                [0, L): a precondition), or NULL for positions 0 .. n_sel-1;
 *                1 <= n_sel <= 32768.
 *   sm_scale in  score scale (usually 1/sqrt(D)).
 *   out      out float32 [Tq][Hq][D]:
 *                out[t][h] = sum_i p_i v[sel[t][i]][h / (Hq/Hkv)],
 *                p = softmax_i(sm_scale * q[t][h] . k[sel[t][i]][...]),
 *                in fp32; chunks of 32 or 64 positions are combined in a fixed
 *                order, so the result is deterministic.
 *   workspace  device scratch of strata_sparse_attention_workspace_size(Tq,
 *              Hq, n_sel) bytes, 256-byte aligned.
 */
size_t strata_sparse_attention_workspace_size(int32_t Tq, int32_t Hq, int32_t n_sel);
int strata_sparse_attention(const uint16_t *q_bf16, int32_t Tq, int32_t Hq, const uint8_t *k_codes,
                            const uint16_t *k_scales, const uint8_t *v_codes, const uint16_t *v_scales, int32_t L,
                            int32_t Hkv, int32_t D, const int32_t *sel, int32_t n_sel, float sm_scale, float *out,
                            void *workspace, size_t workspace_bytes, void *stream);

/* Message describing the last failed call on this thread ("" if none). */
const char *strata_moe_last_error(void);

/*
 * Diagnostics: optional per-kernel device timing, off by default (timers that
 * exist but stay disabled unless asked for: lqnn.cn static review §5.3).
 * While enabled, each kernel the library launches is bracketed by two HIP
 * events recorded on its launch stream (the events are created by the
 * library and reused; no device memory is allocated).
 *
 * strata_moe_timing_enable(on)  discards collected records; on != 0 starts
 *                               recording.  Returns STRATA_OK.
 * strata_moe_timing_query(kernel, launches, total_ms)
 *                               waits for the recorded events and returns the
 *                               number of launches of `kernel` (NULL: all
 *                               kernels) and their summed device time in ms.
 * strata_moe_timing_kernels(names, max_names)
 *                               writes up to max_names distinct kernel names
 *                               (static strings) in first-launch order and
 *                               returns how many there are.
 * Kernel names: router_logits, route_topk, route_xconv, permute_small, permute_hist,
 * permute_scan, permute_scatter, ffn_prep, gemm_gateup, gemm_down,
 * gemv_gateup, gemv_down, combine, decode_route_gateup, decode_down_combine,
 * kv_quantize, attn_partial, attn_merge.
 */
int strata_moe_timing_enable(int32_t on);
int strata_moe_timing_query(const char *kernel, int32_t *launches, double *total_ms);
int32_t strata_moe_timing_kernels(const char **names, int32_t max_names);

#ifdef __cplusplus
}
#endif

#endif /* STRATA_MOE_H */
