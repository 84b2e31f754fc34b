// Router top-k with softmax gating: one wavefront per token.
//
// Each layer's router selects a few experts per token out of a large pool
// ("两天移植，预填充提速8倍：Strata引擎实测" (kongchang.com), section
// "Strata快在哪：不是魔法，是物流", MoE note: 512 experts, about 10 active).
//
// Every lane holds ceil(E/64) logits as order-preserving unsigned keys
// (-0.0 is canonicalised to +0.0 first, so signed zeros tie as under IEEE
// equality); the k winners are the first k in the order (key descending,
// expert index ascending).  A threshold from the lane maxima leaves a few
// candidates, which are ranked against each other in LDS (route_dev.h; many
// equal logits fall back to k rounds of wavefront maxima).  Lane j then owns
// winner j, and the softmax over the k selected logits is a wavefront sum in
// fixed order.
#include <algorithm>

#include "route_dev.h"
#include "tiles_dev.h"

namespace strata {
namespace {

template <int EPL>
__global__ __launch_bounds__(256) void route_topk_kernel(const float *__restrict__ logits, int T,
                                                         int E, int k, int *__restrict__ ids,
                                                         float *__restrict__ w) {
  __shared__ TopkScratch sc[4];
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  wave_route_token<EPL>(logits + (size_t)t * E, E, k, ids + (size_t)t * k, w + (size_t)t * k, sc[threadIdx.x >> 6]);
}

// Routing plus the grouped-GEMM path's conversion of x to fp16: the first
// gridDim.x - nroute workgroups convert x, the other nroute route 4 tokens
// each (the two are independent; sharing one launch saves a kernel boundary
// in the layer call).  The streaming conversion blocks go first so that they
// start together and the routing blocks fill in around them.
template <int EPL>
__global__ __launch_bounds__(256) void route_convert_kernel(const float *__restrict__ logits, int T, int E, int k,
                                                            int *__restrict__ ids, float *__restrict__ w,
                                                            const uint4 *__restrict__ x, uint4 *__restrict__ xq,
                                                            size_t n8, int nroute) {
  const int nconv = gridDim.x - nroute;
  if ((int)blockIdx.x < nconv) {
    convert_x_slots(x, xq, n8, blockIdx.x, nconv);
    return;
  }
  __shared__ TopkScratch sc[4];
  const int t = (blockIdx.x - nconv) * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  wave_route_token<EPL>(logits + (size_t)t * E, E, k, ids + (size_t)t * k, w + (size_t)t * k, sc[threadIdx.x >> 6]);
}

}  // namespace

hipError_t launch_route_convert(const float *logits, int T, int E, int k, int *ids, float *w, const uint16_t *x,
                                uint16_t *xq, size_t n8, hipStream_t s) {
  const int nroute = ceil_div(T, 4);
  // Conversion workgroups: 8 slots (128 bytes of x) per thread each, at most 1024.
  const int nconv = (int)std::max<size_t>(1, std::min<size_t>(1024, (n8 + 2047) / 2048));
  const dim3 grid(nroute + nconv), block(256);
  const uint4 *xs = reinterpret_cast<const uint4 *>(x);
  uint4 *xd = reinterpret_cast<uint4 *>(xq);
  KernelTimer timer("route_xconv", s);
  if (E <= 64)
    route_convert_kernel<1><<<grid, block, 0, s>>>(logits, T, E, k, ids, w, xs, xd, n8, nroute);
  else if (E <= 128)
    route_convert_kernel<2><<<grid, block, 0, s>>>(logits, T, E, k, ids, w, xs, xd, n8, nroute);
  else if (E <= 256)
    route_convert_kernel<4><<<grid, block, 0, s>>>(logits, T, E, k, ids, w, xs, xd, n8, nroute);
  else if (E <= 512)
    route_convert_kernel<8><<<grid, block, 0, s>>>(logits, T, E, k, ids, w, xs, xd, n8, nroute);
  else
    route_convert_kernel<16><<<grid, block, 0, s>>>(logits, T, E, k, ids, w, xs, xd, n8, nroute);
  return hipGetLastError();
}

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
