// Weighted combine of each token's k expert outputs (deterministic form):
//   out[t][n] = sum_{j=0}^{k-1} topk_w[t*k+j] * y[inv_perm[t*k+j]][n],
// summed in j order.  The fused form of the same sum is the down-GEMM
// epilogue; this kernel finishes the layer when the FFN wrote grouped rows.
#include "moe_internal.h"

namespace strata {
namespace {
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ y,
                                                      const int *__restrict__ inv_perm,
                                                      const float *__restrict__ topk_w, int T, int k,
                                                      int H, float *__restrict__ out) {
  const int chunks = (H / 4 + 255) / 256;
  const int t = blockIdx.x / chunks;
  const int n4 = (blockIdx.x - t * chunks) * 256 + threadIdx.x;  // float4 column index
  if (n4 * 4 >= H) return;
  float4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < k; ++j) {
    const int i = inv_perm[(size_t)t * k + j];
    const float w = topk_w[(size_t)t * k + j];
    const float4 v = reinterpret_cast<const float4 *>(y + (size_t)i * H)[n4];
    acc.x += w * v.x;
    acc.y += w * v.y;
    acc.z += w * v.z;
    acc.w += w * v.w;
  }
  reinterpret_cast<float4 *>(out + (size_t)t * H)[n4] = acc;
}

// Fused-combine finish: fp16 y rows in pair order, so the k rows of token t
// are contiguous.  One thread: 8 consecutive features.  All of a thread's
// row loads are issued before the first is used (KMAX >= k of them, rows past
// k repeat row k-1 with weight 0), so that each thread keeps k loads in
// flight.  The rows are read once and out is not read back here, so both go
// through non-temporal accesses (they do not displace other data in the
// caches).  Sum in j order, in fp32.
template <int KMAX>
__global__ __launch_bounds__(256) void combine_pairs_kernel(const uint4 *__restrict__ y16,
                                                            const float *__restrict__ topk_w, int T, int k,
                                                            int H, float4 *__restrict__ out) {
  const int groups = H / 8;
  const long long g = (long long)blockIdx.x * 256 + threadIdx.x;
  if (g >= (long long)T * groups) return;
  const int t = (int)(g / groups), c = (int)(g - (long long)t * groups);
  u32x4_t v[KMAX];
  float w[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const int jj = j < k ? j : k - 1;
    v[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(&y16[((size_t)t * k + jj) * groups + c]));
    w[j] = j < k ? topk_w[(size_t)t * k + jj] : 0.0f;
  }
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const uint32_t d[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const auto h2 = __builtin_bit_cast(_Float16 __attribute__((ext_vector_type(2))), d[q]);
      acc[2 * q] += w[j] * (float)h2.x;
      acc[2 * q + 1] += w[j] * (float)h2.y;
    }
  }
  __builtin_nontemporal_store(f32x4_t{acc[0], acc[1], acc[2], acc[3]}, reinterpret_cast<f32x4_t *>(&out[g * 2]));
  __builtin_nontemporal_store(f32x4_t{acc[4], acc[5], acc[6], acc[7]}, reinterpret_cast<f32x4_t *>(&out[g * 2 + 1]));
}

// Instance KMAX = k for every k up to 16 (no padding rows to load), and
// kMaxTopK above that.
template <int KMAX>
void combine_pairs_for_k(const uint4 *y, const float *topk_w, int T, int k, int H, float4 *out, dim3 grid,
                         hipStream_t s) {
  if constexpr (KMAX < 16) {
    if (k > KMAX) return combine_pairs_for_k<KMAX + 1>(y, topk_w, T, k, H, out, grid, s);
  } else if constexpr (KMAX == 16) {
    if (k > KMAX) return combine_pairs_for_k<kMaxTopK>(y, topk_w, T, k, H, out, grid, s);
  }
  combine_pairs_kernel<KMAX><<<grid, 256, 0, s>>>(y, topk_w, T, k, H, out);
}

}  // namespace

hipError_t launch_combine_pairs(const uint16_t *y16, const float *topk_w, int T, int k, int H, float *out,
                                hipStream_t s) {
  const long long groups = (long long)T * (H / 8);
  KernelTimer timer("combine", s);
  const dim3 grid((unsigned)((groups + 255) / 256));
  combine_pairs_for_k<1>(reinterpret_cast<const uint4 *>(y16), topk_w, T, k, H, reinterpret_cast<float4 *>(out),
                         grid, s);
  return hipGetLastError();
}

hipError_t launch_combine(const float *y, const int *inv_perm, const float *topk_w, int T, int k,
                          int H, float *out, hipStream_t s) {
  const long long blocks = (long long)ceil_div(H / 4, 256) * T;
  KernelTimer timer("combine", s);
  combine_kernel<<<dim3((unsigned)blocks), 256, 0, s>>>(y, inv_perm, topk_w, T, k, H, out);
  return hipGetLastError();
}

}  // namespace strata
