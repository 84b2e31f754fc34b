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
// Large inputs: one wavefront per segment of kPermuteSeg consecutive pairs.
//   1. seg_hist:   hist[e][s] = pairs of expert e in segment s
//   2. seg_scan:   one workgroup turns hist into the exclusive scan over the
//                  (e-major, s-minor) order: base[e][s] = first grouped slot
//                  of expert e's pairs from segment s; also counts/offsets
//   3. seg_scatter: each segment walks its pairs in order from base[.][s]
// Small inputs (<= kPermuteSmallMax pairs): one workgroup does all three.
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

// Wavefront `wave` of the block walks pairs [p0, p1) (at most kPermuteSeg) in
// rounds of 64 and places each at running[e] + rank; running[] lives in LDS.
// All expert ids of the segment are loaded up front so their latency overlaps.
__device__ __forceinline__ void scatter_rounds(const int *__restrict__ ids, int p0, int p1, int E,
                                               int *running, int *__restrict__ perm,
                                               int *__restrict__ inv_perm) {
  constexpr int R = kPermuteSeg / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int nbits = id_bits(E);
  int ev[R];
#pragma unroll
  for (int q = 0; q < R; ++q) {
    const int p = p0 + q * kWave + lane;
    ev[q] = p < p1 ? ids[p] : E;  // sentinel E never matches a real expert
  }
#pragma unroll
  for (int q = 0; q < R; ++q) {
    if (p0 + q * kWave >= p1) break;
    const int p = p0 + q * kWave + lane;
    const int e = ev[q];
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

__global__ __launch_bounds__(256) void seg_hist_kernel(const int *__restrict__ ids, int pairs, int E,
                                                       int nseg, int *__restrict__ hist) {
  constexpr int R = kPermuteSeg / kWave;
  __shared__ int h[4][kMaxExperts];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int s = blockIdx.x * 4 + wave;
  for (int e = lane; e < E; e += kWave) h[wave][e] = 0;
  int ev[R];
  const int p0 = s * kPermuteSeg, p1 = min(pairs, p0 + kPermuteSeg);
#pragma unroll
  for (int q = 0; q < R; ++q) {
    const int p = p0 + q * kWave + lane;
    ev[q] = (s < nseg && p < p1) ? ids[p] : -1;
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < R; ++q)
    if (ev[q] >= 0) atomicAdd(&h[wave][ev[q]], 1);
  __syncthreads();
  if (s < nseg)
    for (int e = lane; e < E; e += kWave) hist[(size_t)e * nseg + s] = h[wave][e];
}

// Exclusive scan of hist (E*nseg ints, e-major) in place by one workgroup:
// passes of 8192 ints are loaded into LDS with coalesced reads, scanned there
// (8 contiguous values per thread, then across threads) and written back.
__global__ __launch_bounds__(1024) void seg_scan_kernel(int *__restrict__ hist, int E, int nseg,
                                                        int pairs, int *__restrict__ counts,
                                                        int *__restrict__ offsets) {
  constexpr int CH = 8192, PER = CH / 1024;
  __shared__ int buf[CH + CH / 32];  // one pad int per 32 breaks the stride-8 bank pattern
  __shared__ int wsum[16];
  const int n = E * nseg;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  auto at = [](int i) { return i + (i >> 5); };
  int carry = 0;
  for (int base = 0; base < n; base += CH) {
    const int m = min(CH, n - base);
    for (int i = tid; i < CH; i += 1024) buf[at(i)] = i < m ? hist[base + i] : 0;
    __syncthreads();
    int v[PER], sum = 0;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      v[q] = buf[at(tid * PER + q)];
      sum += v[q];
    }
    int incl = sum;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int t = __shfl_up(incl, off, kWave);
      if (lane >= off) incl += t;
    }
    if (lane == kWave - 1) wsum[wave] = incl;
    __syncthreads();
    int run = carry + incl - sum;
    int total = 0;
    for (int w2 = 0; w2 < 16; ++w2) {
      if (w2 < wave) run += wsum[w2];
      total += wsum[w2];
    }
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      buf[at(tid * PER + q)] = run;
      run += v[q];
    }
    __syncthreads();
    for (int i = tid; i < m; i += 1024) hist[base + i] = buf[at(i)];
    carry += total;
    __syncthreads();
  }
  for (int e = tid; e < E; e += 1024) {
    const int o0 = hist[(size_t)e * nseg];
    const int o1 = e + 1 < E ? hist[(size_t)(e + 1) * nseg] : pairs;
    offsets[e] = o0;
    counts[e] = o1 - o0;
  }
  if (tid == 0) offsets[E] = pairs;
}

__global__ __launch_bounds__(256) void seg_scatter_kernel(const int *__restrict__ ids, int pairs,
                                                          int E, int nseg,
                                                          const int *__restrict__ base,
                                                          int *__restrict__ perm,
                                                          int *__restrict__ inv_perm) {
  __shared__ int running[4][kMaxExperts];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int s = blockIdx.x * 4 + wave;
  if (s >= nseg) return;  // whole wavefront leaves together; no block barrier below
  for (int e = lane; e < E; e += kWave) running[wave][e] = base[(size_t)e * nseg + s];
  // LDS writes above are read back by other lanes of the same wavefront only.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  const int p0 = s * kPermuteSeg, p1 = min(pairs, p0 + kPermuteSeg);
  scatter_rounds(ids, p0, p1, E, running[wave], perm, inv_perm);
}

// Whole grouping in one workgroup (wavefront 0 does the ordered scatter).
__global__ __launch_bounds__(256) void small_permute_kernel(const int *__restrict__ ids, int pairs,
                                                            int E, int *__restrict__ counts,
                                                            int *__restrict__ offsets,
                                                            int *__restrict__ perm,
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
  if (wave == 0) scatter_rounds(ids, 0, pairs, E, h, perm, inv_perm);
}

}  // namespace

size_t permute_workspace_bytes(long long pairs, int E) {
  if (pairs <= kPermuteSmallMax) return 0;
  const long long nseg = (pairs + kPermuteSeg - 1) / kPermuteSeg;
  return (size_t)((nseg * E * 4 + 255) / 256 * 256);
}

hipError_t launch_permute(const int *ids, int pairs, int E, int *counts, int *offsets, int *perm,
                          int *inv_perm, void *ws, hipStream_t s) {
  if (pairs <= kPermuteSmallMax) {
    KernelTimer timer("permute_small", s);
    small_permute_kernel<<<1, 256, 0, s>>>(ids, pairs, E, counts, offsets, perm, inv_perm);
    return hipGetLastError();
  }
  const int nseg = ceil_div(pairs, kPermuteSeg);
  int *hist = static_cast<int *>(ws);
  const int blocks = ceil_div(nseg, 4);
  {
    KernelTimer timer("permute_hist", s);
    seg_hist_kernel<<<blocks, 256, 0, s>>>(ids, pairs, E, nseg, hist);
  }
  {
    KernelTimer timer("permute_scan", s);
    seg_scan_kernel<<<1, 1024, 0, s>>>(hist, E, nseg, pairs, counts, offsets);
  }
  {
    KernelTimer timer("permute_scatter", s);
    seg_scatter_kernel<<<blocks, 256, 0, s>>>(ids, pairs, E, nseg, hist, perm, inv_perm);
  }
  return hipGetLastError();
}

}  // namespace strata
