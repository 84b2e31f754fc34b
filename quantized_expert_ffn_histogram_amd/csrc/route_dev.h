// Device-side top-k selection of one token's expert logits, shared by the
// routing kernel and the fused decode kernel.  See route.hip for the method.
#pragma once
#include "moe_internal.h"

namespace strata {
namespace {

__device__ __forceinline__ uint32_t orderable(float v) {
  uint32_t b = __float_as_uint(v == 0.0f ? 0.0f : v);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float from_orderable(uint32_t u) {
  uint32_t b = (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u;
  return __uint_as_float(b);
}

// The calling wavefront selects, in order, the `rounds` largest of the E
// logits in `row` (ties to the lower expert index; -0.0 equals +0.0): lane r
// (r < rounds) receives the r-th in my_id / my_val.
template <int EPL>
__device__ __forceinline__ void wave_topk(const float *__restrict__ row, int E, int rounds, int &my_id,
                                          float &my_val) {
  const int lane = threadIdx.x & (kWave - 1);
  // u[i] = orderable value of expert i*64 + lane; 0 = absent or already taken
  // (every finite logit maps above 0).
  // Loads are unconditional (clamped to expert 0) so that all of them are in
  // flight together; absent experts are masked afterwards.
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

// The calling wavefront routes one token: ids[0..k) = the k largest logits in
// order, w = softmax over those k logits (fp32, shifted by the largest).
template <int EPL>
__device__ __forceinline__ void wave_route_token(const float *__restrict__ row, int E, int k, int *__restrict__ ids,
                                                 float *__restrict__ w) {
  const int lane = threadIdx.x & (kWave - 1);
  int my_id;
  float my_val;
  wave_topk<EPL>(row, E, k, my_id, my_val);
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
