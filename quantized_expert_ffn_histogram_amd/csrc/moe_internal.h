// Internal declarations of the gfx950 MoE FFN library: kernel launchers and
// the device-side helpers they share.  Not part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace strata {

// ---------------------------------------------------------------- constants
constexpr int kWave = 64;                 // CDNA wavefront width
constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 32;

// Grouping: pairs handled by one wavefront in the multi-block histogram/scatter.
constexpr int kPermuteSeg = 1024;
// At or below this many pairs the whole grouping runs in one workgroup.
constexpr int kPermuteSmallMax = 1024;

// Grouped GEMM tiling (rows of one expert per tile, K per LDS chunk).
constexpr int kGemmRows = 128;
constexpr int kGemmKChunk = 64;

// GEMV (few pairs per expert): rows of one expert per work entry.
constexpr int kGemvMaxTokens = 16;        // auto path picks GEMV at or below this T
constexpr int kGemvMaxHidden = 4096;

// Fused decode layer (strata_moe_layer at T <= kGemvMaxTokens): top-k per
// token and h of a token's k pairs staged in LDS (k * I fp16 values).
constexpr int kDecodeMaxK = 16;
constexpr int kDecodeMaxKI = 16384;

// One unit of grouped work: `rows` consecutive grouped rows of expert `e`
// starting at grouped row `row0`.
struct Tile {
  int e, row0, rows, pad;
};

struct FfnWeights {
  const uint8_t *gate, *up, *down;
  const uint16_t *gate_s, *up_s, *down_s;
  int E, H, I, g;
  int fmt = 0;  // strata_weight_format: 0 symmetric 4-bit, 1 asymmetric 4-bit, 2 symmetric 5-bit
  // Side data of formats 1 and 2: zero points [E][N][K/g/2] (two per byte)
  // or fifth-bit words [E][N][K/32] (as bytes).
  const uint8_t *gate_x = nullptr, *up_x = nullptr, *down_x = nullptr;
  int tiled = 0;  // packed codes in 32-row x 128-K tiles (packed_offset), else row-major
};

// Byte offset of packed byte `kb` (K index 2*kb) of weight row `row` in a
// matrix of `rb` = K/2 bytes per row; `row` counts the rows of all experts
// (e*N + n; N is a multiple of 32, K of 128).  Row-major: row*rb + kb.
// Tiled: a 32-row block's K/128 tiles of 32 rows x 64 bytes follow one
// another, each row's 64 bytes contiguous inside its tile, so the 64 bytes of
// one 128-wide K stage of 32 rows are one 2 KB run.
__host__ __device__ __forceinline__ size_t packed_offset(size_t row, uint32_t kb, uint32_t rb, bool tiled) {
  return tiled ? ((row >> 5) * (rb >> 6) + (kb >> 6)) * 2048u + (row & 31u) * 64u + (kb & 63u) : row * rb + kb;
}

// ---------------------------------------------------------------- launchers
// Row-major packed codes [rows][K/2] -> the tiled layout of packed_offset.
hipError_t launch_tile_weights(const uint8_t *src, uint8_t *dst, long long rows, int K, hipStream_t s);
hipError_t launch_route(const float *logits, int T, int E, int k, int *ids, float *w,
                        hipStream_t s);
// Router projection logits[t][e] = x[t] . w_router[e] (bf16 in, fp32 out).
hipError_t launch_router_logits(const uint16_t *x, int T, int H, const uint16_t *w_router, int E, float *logits,
                                hipStream_t s);
// Routing plus the conversion of x (bf16 [T][H], n8 = T*H/8) to the grouped
// GEMM's fp16 slot order in xq, in one launch (layer call, GEMM path).
hipError_t launch_route_convert(const float *logits, int T, int E, int k, int *ids, float *w, const uint16_t *x,
                                uint16_t *xq, size_t n8, hipStream_t s);

size_t permute_workspace_bytes(long long pairs, int E);
// With `tiles` non-null (multi-block path only, pairs > kPermuteSmallMax) the
// scan also writes the grouped-GEMM tile lists: tiles sorted by cost,
// by_expert in expert order, meta[0] = their number.
hipError_t launch_permute(const int *ids, int pairs, int E, int *counts, int *offsets,
                          int *perm, int *inv_perm, void *ws, hipStream_t s, Tile *tiles = nullptr,
                          Tile *by_expert = nullptr, int *meta = nullptr);

// Workspace carving for the FFN (activations, h, fp16 y rows, tile list).
struct FfnWorkspace {
  uint16_t *xq;      // fp16 [T][H], fragment slot order (GEMM path)
  uint16_t *h;       // fp16 [pairs][I]
  uint16_t *y16;     // fp16 [pairs][H], pair order (fused combine)
  Tile *tiles;       // GEMM path work lists, [2][tile_cap]: sorted by cost, then in expert order
  long long tile_cap;
  int *meta;         // meta[0] = number of tiles
  size_t bytes;
};
size_t ffn_workspace_bytes(long long T, int k, int E, int H, int I);
FfnWorkspace carve_ffn_workspace(void *base, long long T, int k, int E, int H, int I);

// prepared: xq and the tile lists are already in the workspace (the layer
// call's routing and grouping kernels wrote them); otherwise a prologue
// kernel makes them from x and offsets.
hipError_t launch_ffn_gemm(const uint16_t *x, int T, int k, const FfnWeights &w,
                           const int *offsets, const int *perm, const float *topk_w,
                           float *y_or_out, const FfnWorkspace &ws, hipStream_t s, bool prepared = false);
hipError_t launch_ffn_gemv(const uint16_t *x, int T, int k, const FfnWeights &w,
                           const int *offsets, const int *perm, const float *topk_w,
                           float *y_or_out, const FfnWorkspace &ws, hipStream_t s);

bool gemv_supported(int T, int H, int I);

// Whole layer for a decode batch in two kernels (route + gate/up, grouping +
// down + combine); fills every output of route, permute and the fused ffn.
bool decode_layer_supported(int T, int E, int k, int H, int I);
hipError_t launch_decode_layer(const float *logits, const uint16_t *x, int T, int k, const FfnWeights &w,
                               int *ids, float *topk_w, int *counts, int *offsets, int *perm, int *inv_perm,
                               float *out, const FfnWorkspace &ws, hipStream_t s);

hipError_t launch_combine(const float *y, const int *inv_perm, const float *topk_w, int T,
                          int k, int H, float *out, hipStream_t s);
// out[t] = sum_j topk_w[t*k+j] * y16[t*k+j] (fp16 rows in pair order), j in order.
hipError_t launch_combine_pairs(const uint16_t *y16, const float *topk_w, int T, int k, int H, float *out,
                                hipStream_t s);

// 4-bit KV cache (kv.hip): per-head symmetric codes of key/value vectors and
// attention of queries over selected cache rows.
bool kv_shape_supported(int Hkv, int D);
// With x2 non-null a second tensor of the same tokens (values beside keys) is
// encoded in the same launch into codes2 / scale2.
hipError_t launch_kv_quantize(const uint16_t *x, int T, int Hkv, const int *slots, int L, uint8_t *codes,
                              uint16_t *scale, hipStream_t s, const uint16_t *x2 = nullptr,
                              uint8_t *codes2 = nullptr, uint16_t *scale2 = nullptr);
size_t attn_workspace_bytes(int Tq, int Hq, int n_sel);
hipError_t launch_sparse_attention(const uint16_t *q, int Tq, int Hq, const uint8_t *kc, const uint16_t *ks,
                                   const uint8_t *vc, const uint16_t *vs, int L, int Hkv, const int *sel,
                                   int n_sel, float sm_scale, float *out, void *ws, hipStream_t s);

inline int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

// ---------------------------------------------------------------- wavefront reductions
// Reduce within each row of 16 lanes with DPP (quad_perm [1,0,3,2], [2,3,0,1],
// row_ror 4, row_ror 8), then combine the four row results read from lanes
// 0, 16, 32, 48.  The result is wavefront-uniform and its order of operations
// is fixed.
#define STRATA_DPP_ROW_REDUCE(v, OP, T)                                                           \
  do {                                                                                            \
    v = OP(v, (T)__builtin_amdgcn_update_dpp(0, (int)(v), 0xB1, 0xF, 0xF, false));               \
    v = OP(v, (T)__builtin_amdgcn_update_dpp(0, (int)(v), 0x4E, 0xF, 0xF, false));               \
    v = OP(v, (T)__builtin_amdgcn_update_dpp(0, (int)(v), 0x124, 0xF, 0xF, false));              \
    v = OP(v, (T)__builtin_amdgcn_update_dpp(0, (int)(v), 0x128, 0xF, 0xF, false));              \
  } while (0)

__device__ __forceinline__ uint32_t umax32(uint32_t a, uint32_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint32_t umin32(uint32_t a, uint32_t b) { return a < b ? a : b; }

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  STRATA_DPP_ROW_REDUCE(v, umax32, uint32_t);
  const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
  const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
  return umax32(umax32(a, b), umax32(c, d));
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  STRATA_DPP_ROW_REDUCE(v, umin32, uint32_t);
  const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
  const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
  return umin32(umin32(a, b), umin32(c, d));
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float wave_sum_f32(float v) {
  v = v + dpp_f32<0xB1>(v);
  v = v + dpp_f32<0x4E>(v);
  v = v + dpp_f32<0x124>(v);
  v = v + dpp_f32<0x128>(v);
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (a + b) + (c + d);
}

// Optional per-kernel timing (see timing.hip).  A KernelTimer brackets one
// kernel launch with events on its stream while timing is enabled.
void timing_begin(const char *name, hipStream_t s);
void timing_end(hipStream_t s);
int timing_enable(int on);
int timing_query(const char *name, int *launches, double *total_ms);
int timing_names(const char **names, int max_names);

struct KernelTimer {
  hipStream_t s;
  KernelTimer(const char *name, hipStream_t st) : s(st) { timing_begin(name, st); }
  ~KernelTimer() { timing_end(s); }
};

}  // namespace strata
