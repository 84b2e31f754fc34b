// Router top-k with softmax gating: one wavefront per token.
//
// Each layer's router selects a few experts per token out of a large pool
// ("两天移植，预填充提速8倍：Strata引擎实测" (kongchang.com), section
// "Strata快在哪：不是魔法，是物流", MoE note: 512 experts, about 10 active).
//
// Every lane holds ceil(E/64) logits as 64-bit keys
//     key = orderable(logit) << 32 | (0xFFFFFFFF - e)
// so that the unsigned maximum is the largest logit and, among equal logits,
// the lowest expert index.  -0.0 is canonicalised to +0.0 first so that signed
// zeros tie (IEEE equality).  k rounds of (per-lane max, wavefront max,
// remove the winner) give the ordered top-k; lane j then owns winner j and the
// softmax over the k selected logits is a wavefront sum.
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

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint64_t o = __shfl_xor(v, off, kWave);
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

template <int EPL>
__global__ __launch_bounds__(256) void route_topk_kernel(const float *__restrict__ logits, int T,
                                                         int E, int k, int *__restrict__ ids,
                                                         float *__restrict__ w) {
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float *row = logits + (size_t)t * E;

  uint64_t key[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = i * kWave + lane;
    key[i] = 0;  // below every real key: never selected while k <= E
    if (e < E) key[i] = ((uint64_t)orderable(row[e]) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e);
  }

  int my_id = 0;
  float my_val = 0.0f;
  for (int r = 0; r < k; ++r) {
    uint64_t best = key[0];
#pragma unroll
    for (int i = 1; i < EPL; ++i) best = key[i] > best ? key[i] : best;
    best = wave_max_u64(best);
    const int e = (int)(0xFFFFFFFFu - (uint32_t)best);
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (i * kWave + lane == e) key[i] = 0;
    if (lane == r) {
      my_id = e;
      my_val = from_orderable((uint32_t)(best >> 32));
    }
  }

  const float m = __shfl(my_val, 0, kWave);
  const float z = lane < k ? expf(my_val - m) : 0.0f;
  const float s = wave_sum(z);
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
