// Router top-k with softmax gating: one wavefront per token.
//
// Each layer's router selects a few experts per token out of a large pool
// ("两天移植，预填充提速8倍：Strata引擎实测" (kongchang.com), section
// "Strata快在哪：不是魔法，是物流", MoE note: 512 experts, about 10 active).
//
// Every lane holds ceil(E/64) logits as order-preserving unsigned keys
// (-0.0 is canonicalised to +0.0 first, so signed zeros tie as under IEEE
// equality).  Each of k rounds takes the wavefront maximum key and then the
// minimum expert index among the lanes holding it (ties go to the lowest
// index; with a single holder that is the holder's own candidate), and
// removes the winner.  Lane j then owns winner j, and the softmax
// over the k selected logits is a wavefront sum in fixed order.
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

template <int EPL>
__global__ __launch_bounds__(256) void route_topk_kernel(const float *__restrict__ logits, int T,
                                                         int E, int k, int *__restrict__ ids,
                                                         float *__restrict__ w) {
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float *row = logits + (size_t)t * E;

  // u[i] = orderable value of expert i*64 + lane; 0 = absent or already taken
  // (every finite logit maps above 0).
  uint32_t u[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = i * kWave + lane;
    u[i] = e < E ? orderable(row[e]) : 0u;
  }

  int my_id = 0;
  float my_val = 0.0f;
  for (int r = 0; r < k; ++r) {
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

  const float m = __shfl(my_val, 0, kWave);
  const float z = lane < k ? expf(my_val - m) : 0.0f;
  const float s = wave_sum_f32(z);
  if (lane < k) {
    ids[(size_t)t * k + lane] = my_id;
    w[(size_t)t * k + lane] = z / s;
  }
}

}  // namespace

hipError_t launch_route(const float *logits, int T, int E, int k, int *ids, float *w,
                        hipStream_t s) {
  const dim3 grid(ceil_div(T, 4)), block(256);
  KernelTimer timer("route_topk", s);
  if (E <= 64)
    route_topk_kernel<1><<<grid, block, 0, s>>>(logits, T, E, k, ids, w);
  else if (E <= 128)
    route_topk_kernel<2><<<grid, block, 0, s>>>(logits, T, E, k, ids, w);
  else if (E <= 256)
    route_topk_kernel<4><<<grid, block, 0, s>>>(logits, T, E, k, ids, w);
  else if (E <= 512)
    route_topk_kernel<8><<<grid, block, 0, s>>>(logits, T, E, k, ids, w);
  else
    route_topk_kernel<16><<<grid, block, 0, s>>>(logits, T, E, k, ids, w);
  return hipGetLastError();
}

}  // namespace strata
