// Grouping of (token, slot) pairs by expert: histogram, exclusive scan and a
// stable counting-sort scatter.
//
// Tokens routed to the same expert are processed as one batch so that its
// weights serve all of them ("两天移植，预填充提速8倍：Strata引擎实测"
// (kongchang.com), section "Strata快在哪：不是魔法，是物流").  The grouped
// order is the stable order of the pair index p = t*k + j inside each expert,
// so every output is bit-exact and independent of scheduling:
//   * counts come from LDS atomic increments (an order-free sum);
//   * a pair's slot is its rank among equal experts within its wavefront
//     round (ballot over the expert id's bits) plus a running per-expert
//     counter kept in LDS and advanced in round order.
//
// Large inputs: one workgroup (4 wavefronts) per segment of kPermuteSeg
// consecutive pairs.
//   1. seg_hist:    hist[s][e] = pairs of expert e in segment s
//   2. seg_scan:    thread e turns column e of hist into the exclusive prefix
//                   over segments, then one block scan over experts gives
//                   counts/offsets: the first grouped slot of expert e's pairs
//                   from segment s is offsets[e] + hist[s][e]
//   3. seg_scatter: each wavefront counts its quarter of the segment, the
//                   quarters' counts are prefix-summed per expert, and every
//                   wavefront then places its pairs in order from there
// Small inputs (<= kPermuteSmallMax pairs): one workgroup does all three.
#include "permute_dev.h"
#include "tiles_dev.h"

namespace strata {
namespace {

__global__ __launch_bounds__(256) void seg_hist_kernel(const int *__restrict__ ids, int pairs, int E,
                                                       int *__restrict__ hist) {
  constexpr int R = kPermuteSeg / 256;
  __shared__ int h[kMaxExperts];
  const int tid = threadIdx.x, s = blockIdx.x;
  const int p0 = s * kPermuteSeg, p1 = min(pairs, p0 + kPermuteSeg);
  int ev[R];
#pragma unroll
  for (int q = 0; q < R; ++q) {
    const int p = p0 + q * 256 + tid;
    ev[q] = p < p1 ? ids[p] : -1;
  }
  for (int e = tid; e < E; e += 256) h[e] = 0;
  __syncthreads();
#pragma unroll
  for (int q = 0; q < R; ++q)
    if (ev[q] >= 0) atomicAdd(&h[ev[q]], 1);
  __syncthreads();
  for (int e = tid; e < E; e += 256) hist[(size_t)s * E + e] = h[e];
}

// One workgroup of 1024 threads (E <= 1024): thread e scans column e of hist
// (segments in order, batches of 32 loads in flight), then the expert totals
// are scanned across the workgroup.
// With `tiles` non-null it also builds the grouped-GEMM tile lists from the
// offsets (the layer call's GEMM path, which then needs no prologue kernel).
__global__ __launch_bounds__(1024) void seg_scan_kernel(int *__restrict__ hist, int E, int nseg, int pairs,
                                                        int *__restrict__ counts, int *__restrict__ offsets,
                                                        Tile *__restrict__ tiles, Tile *__restrict__ by_expert,
                                                        int *__restrict__ meta) {
  constexpr int B = 32;
  __shared__ int wsum[16];
  __shared__ int soff[kMaxExperts + 1];
  __shared__ unsigned long long part[1024];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int total = 0;
  if (tid < E) {
    for (int s0 = 0; s0 < nseg; s0 += B) {
      int v[B];
#pragma unroll
      for (int i = 0; i < B; ++i) v[i] = s0 + i < nseg ? hist[(size_t)(s0 + i) * E + tid] : 0;
#pragma unroll
      for (int i = 0; i < B; ++i) {
        if (s0 + i < nseg) hist[(size_t)(s0 + i) * E + tid] = total;
        total += v[i];
      }
    }
  }
  int incl = total;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int t = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += t;
  }
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();
  int run = incl - total;
  for (int w2 = 0; w2 < wave; ++w2) run += wsum[w2];
  if (tid < E) {
    offsets[tid] = run;
    counts[tid] = total;
    soff[tid] = run;
  }
  if (tid == 0) {
    offsets[E] = pairs;
    soff[E] = pairs;
  }
  if (tiles != nullptr) {
    __syncthreads();
    plan_tiles(soff, E, tiles, by_expert, meta, part);
  }
}

// Segment s: wavefront w owns pairs [p0 + w*Q, p0 + (w+1)*Q), Q = kPermuteSeg/4.
__global__ __launch_bounds__(256) void seg_scatter_kernel(const int *__restrict__ ids, int pairs, int E,
                                                          const int *__restrict__ hist,
                                                          const int *__restrict__ offsets,
                                                          int *__restrict__ perm, int *__restrict__ inv_perm) {
  constexpr int Q = kPermuteSeg / 4;
  __shared__ int cnt[4][kMaxExperts];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, s = blockIdx.x;
  const int q0 = s * kPermuteSeg + wave * Q, q1 = min(pairs, q0 + Q);
  int ev[Q / kWave];
#pragma unroll
  for (int r = 0; r < Q / kWave; ++r) {
    const int p = q0 + r * kWave + lane;
    ev[r] = p < q1 ? ids[p] : -1;
  }
  for (int e = lane; e < E; e += kWave) cnt[wave][e] = 0;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int r = 0; r < Q / kWave; ++r)
    if (ev[r] >= 0) atomicAdd(&cnt[wave][ev[r]], 1);
  __syncthreads();
  // Per expert: first slot of each quarter = offsets[e] + hist[s][e] + earlier quarters.
  for (int e = tid; e < E; e += 256) {
    int run = offsets[e] + hist[(size_t)s * E + e];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int c = cnt[w][e];
      cnt[w][e] = run;
      run += c;
    }
  }
  __syncthreads();
  scatter_rounds(ev, q0, q1, E, cnt[wave], perm, inv_perm);
}

// Whole grouping in one workgroup.
__global__ __launch_bounds__(256) void small_permute_kernel(const int *__restrict__ ids, int pairs,
                                                            int E, int *__restrict__ counts,
                                                            int *__restrict__ offsets,
                                                            int *__restrict__ perm,
                                                            int *__restrict__ inv_perm) {
  group_small(ids, pairs, E, counts, offsets, perm, inv_perm);
}

}  // namespace

size_t permute_workspace_bytes(long long pairs, int E) {
  if (pairs <= kPermuteSmallMax) return 0;
  const long long nseg = (pairs + kPermuteSeg - 1) / kPermuteSeg;
  return (size_t)((nseg * E * 4 + 255) / 256 * 256);
}

hipError_t launch_permute(const int *ids, int pairs, int E, int *counts, int *offsets, int *perm,
                          int *inv_perm, void *ws, hipStream_t s, Tile *tiles, Tile *by_expert, int *meta) {
  if (pairs <= kPermuteSmallMax) {
    if (tiles != nullptr) return hipErrorInvalidValue;  // the tile lists come from the multi-block scan only
    KernelTimer timer("permute_small", s);
    small_permute_kernel<<<1, 256, 0, s>>>(ids, pairs, E, counts, offsets, perm, inv_perm);
    return hipGetLastError();
  }
  const int nseg = ceil_div(pairs, kPermuteSeg);
  int *hist = static_cast<int *>(ws);
  {
    KernelTimer timer("permute_hist", s);
    seg_hist_kernel<<<nseg, 256, 0, s>>>(ids, pairs, E, hist);
  }
  {
    KernelTimer timer("permute_scan", s);
    seg_scan_kernel<<<1, 1024, 0, s>>>(hist, E, nseg, pairs, counts, offsets, tiles, by_expert, meta);
  }
  {
    KernelTimer timer("permute_scatter", s);
    seg_scatter_kernel<<<nseg, 256, 0, s>>>(ids, pairs, E, hist, offsets, perm, inv_perm);
  }
  return hipGetLastError();
}

}  // namespace strata
