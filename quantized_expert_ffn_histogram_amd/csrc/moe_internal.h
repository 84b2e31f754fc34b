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
constexpr int kGemmKChunk = 128;
constexpr int kGateUpColsPerWG = 128;     // h columns per workgroup (gate+up: 256 B rows)
constexpr int kDownColsPerWG = 256;       // output columns per workgroup

// GEMV (few pairs per expert): rows of one expert per work entry.
constexpr int kGemvRows = 4;
constexpr int kGemvMaxTokens = 16;        // auto path picks GEMV at or below this T
constexpr int kGemvMaxHidden = 4096;
constexpr int kGemvDownRowsPerWG = 8;
constexpr int kGemvGateUpColsPerWG = 16;

// One unit of grouped work: `rows` consecutive grouped rows of expert `e`
// starting at grouped row `row0`.
struct Tile {
  int e, row0, rows, pad;
};

struct FfnWeights {
  const uint8_t *gate, *up, *down;
  const uint16_t *gate_s, *up_s, *down_s;
  int E, H, I, g;
};

// ---------------------------------------------------------------- launchers
hipError_t launch_route(const float *logits, int T, int E, int k, int *ids, float *w,
                        hipStream_t s);

size_t permute_workspace_bytes(long long pairs, int E);
hipError_t launch_permute(const int *ids, int pairs, int E, int *counts, int *offsets,
                          int *perm, int *inv_perm, void *ws, hipStream_t s);

// Workspace carving for the FFN (h, tile list, counters).
struct FfnWorkspace {
  uint16_t *h;       // fp16 [pairs][I]
  Tile *tiles;       // grouped-work list
  int *meta;         // meta[0] = number of tiles
  size_t bytes;
};
size_t ffn_workspace_bytes(long long pairs, int E, int H, int I);
FfnWorkspace carve_ffn_workspace(void *base, long long pairs, int E, int H, int I);

hipError_t launch_ffn_gemm(const uint16_t *x, int T, int k, const FfnWeights &w,
                           const int *offsets, const int *perm, const float *topk_w,
                           float *y_or_out, const FfnWorkspace &ws, hipStream_t s);
hipError_t launch_ffn_gemv(const uint16_t *x, int T, int k, const FfnWeights &w,
                           const int *offsets, const int *perm, const float *topk_w,
                           float *y_or_out, const FfnWorkspace &ws, hipStream_t s);

hipError_t launch_combine(const float *y, const int *inv_perm, const float *topk_w, int T,
                          int k, int H, float *out, hipStream_t s);
hipError_t launch_plan(const int *offsets, int E, int rows_per_tile, Tile *tiles, int *meta,
                       hipStream_t s);
hipError_t launch_zero(float *p, size_t n, hipStream_t s);

inline int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

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
