// Device-side top-k selection of one token's expert logits, shared by the
// routing kernel and the fused decode kernel.  See route.hip for the method.
#pragma once
#include "moe_internal.h"

namespace strata {
namespace {

// Order-preserving unsigned key of a logit (-0.0 canonicalised to +0.0).
// Every value maps to a key >= 1 (the one NaN pattern that would map to 0 is
// raised to 1), so that key 0 can mark an absent expert.
__device__ __forceinline__ uint32_t orderable(float v) {
  uint32_t b = __float_as_uint(v == 0.0f ? 0.0f : v);
  const uint32_t o = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return o ? o : 1u;
}

__device__ __forceinline__ float from_orderable(uint32_t u) {
  uint32_t b = (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u;
  return __uint_as_float(b);
}

// Per-wavefront LDS scratch of the selection below.
struct TopkScratch {
  uint64_t cand[64];         // candidates as (key << 32) | ~expert, zero-padded to a multiple of 8
  uint64_t win[kMaxTopK];    // the selected candidates in rank order
};

// Selection by repeated maxima: each of `rounds` rounds takes the largest
// remaining key (ties to the lowest expert index) and removes it.  Exact for
// any input; used when the threshold below leaves more than 64 candidates
// (many equal logits).
template <int EPL>
__device__ __forceinline__ void topk_by_rounds(uint32_t (&u)[EPL], int rounds, int &my_id, float &my_val) {
  const int lane = threadIdx.x & (kWave - 1);
  for (int r = 0; r < rounds; ++r) {
    // Lane's best: largest value, lowest index among equals (smallest i).
    uint32_t best = u[0];
    int bi = 0;
#pragma unroll
    for (int i = 1; i < EPL; ++i)
      if (u[i] > best) {
        best = u[i];
        bi = i;
      }
    const uint32_t gmax = wave_max_u32(best);
    // Usually one lane holds the maximum: its lowest-index candidate wins.
    // Equal maxima in several lanes take the minimum index over those lanes.
    const uint64_t holders = __ballot(best == gmax);
    int e;
    if (__popcll(holders) == 1) {
      const int wl = __ffsll((long long)holders) - 1;
      e = __builtin_amdgcn_readlane(bi, wl) * kWave + wl;
    } else {
      const uint32_t cand = best == gmax ? (uint32_t)(bi * kWave + lane) : 0xFFFFFFFFu;
      e = (int)wave_min_u32(cand);
    }
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (i * kWave + lane == e) u[i] = 0u;
    if (lane == r) {
      my_id = e;
      my_val = from_orderable(gmax);
    }
  }
}

// The calling wavefront selects, in order, the `rounds` largest of the E
// logits in `row` (ties to the lower expert index; -0.0 equals +0.0): lane r
// (r < rounds) receives the r-th in my_id / my_val.  `sc` is this
// wavefront's own scratch.
//
// The order is the total order of (key descending, index ascending), so the
// result is unique and the method below only has to reach it with little
// arithmetic.  With each lane holding ceil(E/64) keys:
//   1. P = the largest value whose low 16 bits are zero such that at least
//      `rounds` lane maxima are >= P (bitwise search over the 16 high bits,
//      one ballot per bit).  At least `rounds` keys are >= P, so the
//      rounds-th largest key, and with it every selected key, is >= P.
//   2. The keys >= P (typically a dozen or two) are compacted into LDS in
//      ballot order; each such candidate's rank is the number of candidates
//      ahead of it in the total order, and rank r < rounds is winner r.
// More than 64 candidates (many equal logits) fall back to repeated maxima.
template <int EPL>
__device__ __forceinline__ void wave_topk(const float *__restrict__ row, int E, int rounds, int &my_id, float &my_val,
                                          TopkScratch &sc) {
  const int lane = threadIdx.x & (kWave - 1);
  // u[i] = orderable value of expert i*64 + lane; 0 = absent.  Loads are
  // unconditional (clamped to expert 0) so that all of them are in flight
  // together; absent experts are masked afterwards.
  float v[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = i * kWave + lane;
    v[i] = row[e < E ? e : 0];
  }
  uint32_t u[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) u[i] = i * kWave + lane < E ? orderable(v[i]) : 0u;

  my_id = 0;
  my_val = 0.0f;
  uint32_t m = u[0];
#pragma unroll
  for (int i = 1; i < EPL; ++i) m = umax32(m, u[i]);
  uint32_t P = 0;
#pragma unroll
  for (int b = 31; b >= 16; --b) {
    const uint32_t c = P | (1u << b);
    if (__popcll(__ballot(m >= c)) >= rounds) P = c;
  }
  P = P ? P : 1u;  // absent experts (key 0) are never candidates

  int pos[EPL];
  int n = 0;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const uint64_t mk = __ballot(u[i] >= P);
    pos[i] = n + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mk >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mk, 0u));
    n += __popcll(mk);
  }
  if (n > kWave) {
    topk_by_rounds<EPL>(u, rounds, my_id, my_val);
    return;
  }
#pragma unroll
  for (int i = 0; i < EPL; ++i)
    if (u[i] >= P) sc.cand[pos[i]] = ((uint64_t)u[i] << 32) | (uint32_t)~(uint32_t)(i * kWave + lane);
  const int npad = (n + 7) & ~7;
  if (lane >= n && lane < npad) sc.cand[lane] = 0;
  asm volatile("" ::: "memory");
  __builtin_amdgcn_wave_barrier();  // a wavefront's LDS operations complete in order
  asm volatile("" ::: "memory");
  const uint64_t mine = lane < n ? sc.cand[lane] : 0;
  int rank = 0;
  for (int c = 0; c < npad; c += 8) {
    uint64_t o[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) o[q] = sc.cand[c + q];
#pragma unroll
    for (int q = 0; q < 8; ++q) rank += o[q] > mine ? 1 : 0;
  }
  if (lane < n && rank < rounds) sc.win[rank] = mine;
  asm volatile("" ::: "memory");
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
  if (lane < rounds) {
    const uint64_t wv = sc.win[lane];
    my_id = (int)~(uint32_t)wv;
    my_val = from_orderable((uint32_t)(wv >> 32));
  }
}

// The calling wavefront routes one token: ids[0..k) = the k largest logits in
// order, w = softmax over those k logits (fp32, shifted by the largest).
template <int EPL>
__device__ __forceinline__ void wave_route_token(const float *__restrict__ row, int E, int k, int *__restrict__ ids,
                                                 float *__restrict__ w, TopkScratch &sc) {
  const int lane = threadIdx.x & (kWave - 1);
  int my_id;
  float my_val;
  wave_topk<EPL>(row, E, k, my_id, my_val, sc);
  const float m = __shfl(my_val, 0, kWave);
  const float z = lane < k ? expf(my_val - m) : 0.0f;
  const float s = wave_sum_f32(z);
  if (lane < k) {
    ids[lane] = my_id;
    w[lane] = z / s;
  }
}

}  // namespace
}  // namespace strata
