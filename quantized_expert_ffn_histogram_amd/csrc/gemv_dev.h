// Device-side pieces of the GEMV expert FFN (nibble unpacking into fp16
// pairs, dot products with the exact offset correction), shared by the GEMV
// kernels and the fused decode kernels.  See ffn_gemv.hip for the method.
#pragma once
#include "moe_internal.h"

namespace strata {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ half2_t magic_pair(uint32_t d, int m) {
  return __builtin_bit_cast(half2_t, ((d >> (4 * m)) & 0x000F000Fu) | 0x64006400u);
}

// 8 consecutive K values as fp16 pairs in slot order (k+m, k+m+4), m = 0..3.
__device__ __forceinline__ void bf16x8_pairs(uint4 v, half2_t *o) {
  auto lo = [](uint32_t d) { return __uint_as_float(d << 16); };
  auto hi = [](uint32_t d) { return __uint_as_float(d & 0xFFFF0000u); };
  o[0] = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_pkrtz(lo(v.x), lo(v.z)));
  o[1] = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_pkrtz(hi(v.x), hi(v.z)));
  o[2] = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_pkrtz(lo(v.y), lo(v.w)));
  o[3] = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_pkrtz(hi(v.y), hi(v.w)));
}

__device__ __forceinline__ void f16x8_pairs(uint4 v, half2_t *o) {
  o[0] = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(v.z, v.x, 0x05040100u));
  o[1] = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(v.z, v.x, 0x07060302u));
  o[2] = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(v.w, v.y, 0x05040100u));
  o[3] = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(v.w, v.y, 0x07060302u));
}

__device__ __forceinline__ float pair_sum(half2_t p) { return (float)p.x + (float)p.y; }

template <int W>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int off = W / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// sum over this lane's 32 K values of x * q * s, from 16 bytes of packed row.
__device__ __forceinline__ float dot32(const uint4 wq, const half2_t *xp, float xsum, float s) {
  float acc = 0.0f;
  const uint32_t d[4] = {wq.x, wq.y, wq.z, wq.w};
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int m = 0; m < 4; ++m) acc = __builtin_amdgcn_fdot2(xp[4 * q + m], magic_pair(d[q], m), acc, false);
  return s * (acc - 1032.0f * xsum);
}

__device__ __forceinline__ float half_bits_to_float(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

// Makes the compiler treat v as redefined here: it waits for v's load at this
// point (so loads issued together are waited for together), and work derived
// from v (the nibble unpacking) stays inside the row loop instead of being
// hoisted out and held in registers for every row.
__device__ __forceinline__ void opaque(uint4 &v) {
  asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
}

}  // namespace
}  // namespace strata
