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
 * Group-quantized int4 expert weights (all device pointers, caller-owned).
 *
 * Each matrix W[N][K] (gate, up: N = I, K = H; down: N = H, K = I) holds
 * symmetric 4-bit codes q in [-8, 7], K-contiguous rows, two codes per byte:
 * byte j of a row = u(2j) | u(2j+1) << 4 with offset-binary nibble u = q + 8
 * (even K index in the low nibble).  One IEEE fp16 scale per g consecutive K
 * elements: W[n][kk] = q[n][kk] * scale[n][kk / g].
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
 *                 strata_moe_workspace_size(T, E, k, ...) bytes.
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
 *   x_bf16    in  bfloat16 bits [T][H] token activations.  Values must lie in
 *                 the fp16 finite range (|x| <= 65504); the expert matmuls
 *                 run with fp16 operands and fp32 accumulation.
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
 * strata_moe_combine - weighted sum of each token's expert outputs.
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
 * Bytes of device workspace that strata_moe_permute, strata_moe_ffn and
 * strata_moe_layer need for this shape (the ffn's regions plus the grouping
 * histogram's, which strata_moe_layer keeps apart).  Returns 0 for invalid
 * sizes.
 */
size_t strata_moe_workspace_size(int32_t T, int32_t E, int32_t k, int32_t H,
                                 int32_t I, int32_t g);

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
 * gemv_gateup, gemv_down, combine, decode_route_gateup, decode_down_combine.
 */
int strata_moe_timing_enable(int32_t on);
int strata_moe_timing_query(const char *kernel, int32_t *launches, double *total_ms);
int32_t strata_moe_timing_kernels(const char **names, int32_t max_names);

#ifdef __cplusplus
}
#endif

#endif /* STRATA_MOE_H */
