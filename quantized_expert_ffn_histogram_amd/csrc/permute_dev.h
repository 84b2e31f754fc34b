// Device-side pieces of the grouping step (histogram, scan and stable
// scatter of (token, slot) pairs by expert) shared by the grouping kernels and
// the fused decode kernel.  See permute.hip for the method.
#pragma once
#include "moe_internal.h"

namespace strata {
namespace {

__device__ __forceinline__ uint64_t lanemask_lt(int lane) {
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Lanes of this wavefront whose `key` equals mine (key < 2^nbits).
__device__ __forceinline__ uint64_t match_any(int key, int nbits) {
  uint64_t m = __ballot(1);
  for (int b = 0; b < nbits; ++b) {
    const int bit = (key >> b) & 1;
    const uint64_t bb = __ballot(bit);
    m &= bit ? bb : ~bb;
  }
  return m;
}

__device__ __forceinline__ int id_bits(int E) { return 32 - __clz(E); }  // bits of E (sentinel)

// The calling wavefront places pairs [p0, p1) (at most kPermuteSeg, expert
// ids preloaded in ev: pair p0 + q*64 + lane in ev[q], -1 past p1) in rounds
// of 64: each goes to running[e] + its rank among equal experts in the round;
// running[] lives in LDS and is advanced by the round's last lane of each
// expert.
template <int R>
__device__ __forceinline__ void scatter_rounds(const int (&ev)[R], int p0, int p1, int E, int *running,
                                               int *__restrict__ perm, int *__restrict__ inv_perm) {
  const int lane = threadIdx.x & (kWave - 1);
  const int nbits = id_bits(E);
#pragma unroll
  for (int q = 0; q < R; ++q) {
    if (p0 + q * kWave >= p1) break;
    const int p = p0 + q * kWave + lane;
    const int e = ev[q] >= 0 ? ev[q] : E;  // sentinel E never matches a real expert
    const uint64_t same = match_any(e, nbits);
    const int rank = __popcll(same & lanemask_lt(lane));
    const bool last = (same >> lane) == 1ull;  // highest lane of my group
    if (p < p1) {
      const int old = running[e];
      const int dst = old + rank;
      perm[dst] = p;
      inv_perm[p] = dst;
      if (last) running[e] = old + __popcll(same);
    }
    // Keep the next round's LDS reads after this round's counter updates.
    __builtin_amdgcn_wave_barrier();
  }
}

// Whole grouping of `pairs` <= kPermuteSmallMax pairs in one workgroup of 256
// threads (wavefront 0 does the ordered scatter).  `ids` may point to global
// or LDS memory; every thread of the workgroup must call this.
__device__ __forceinline__ void group_small(const int *ids, int pairs, int E, int *__restrict__ counts,
                                            int *__restrict__ offsets, int *__restrict__ perm,
                                            int *__restrict__ inv_perm) {
  __shared__ int h[kMaxExperts];
  __shared__ int wsum[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < E; e += 256) h[e] = 0;
  __syncthreads();
  for (int p = tid; p < pairs; p += 256) atomicAdd(&h[ids[p]], 1);
  __syncthreads();
  // Exclusive scan over E <= 1024 experts: thread tid owns experts [4*tid, 4*tid+4).
  int c[4], sum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = 4 * tid + i;
    c[i] = e < E ? h[e] : 0;
    sum += c[i];
  }
  int incl = sum;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int v = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += v;
  }
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();
  int run = incl - sum;
  for (int w2 = 0; w2 < wave; ++w2) run += wsum[w2];
  __syncthreads();  // every h[] read above is done before h[] becomes the running slot
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = 4 * tid + i;
    if (e < E) {
      offsets[e] = run;
      counts[e] = c[i];
      h[e] = run;
    }
    run += c[i];
  }
  if (tid == 0) offsets[E] = pairs;
  __syncthreads();
  if (wave == 0) {
    int ev[kPermuteSmallMax / kWave];
#pragma unroll
    for (int q = 0; q < kPermuteSmallMax / kWave; ++q) {
      const int p = q * kWave + lane;
      ev[q] = p < pairs ? ids[p] : -1;
    }
    scatter_rounds(ev, 0, pairs, E, h, perm, inv_perm);
  }
}

}  // namespace
}  // namespace strata
