// Device-side pieces of the GEMV expert FFN (nibble unpacking into fp16
// pairs, dot products with the exact offset correction), shared by the GEMV
// kernels and the fused decode kernels.  See ffn_gemv.hip for the method.
#pragma once
#include "moe_internal.h"

namespace strata {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// (a & m) | o as one v_and_or_b32, m in an SGPR and o in a VGPR (one
// scalar operand per VOP3 here); left to itself the compiler emits a
// separate and and or with literal operands.  The asm is volatile: as a
// plain asm the compiler hoists these ahead of their uses and holds the
// results in registers.
__device__ __forceinline__ uint32_t and_or_sv(uint32_t a, uint32_t m, uint32_t o) {
  uint32_t r;
  asm volatile("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(m), "v"(o));
  return r;
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

__device__ __forceinline__ float pair_sum(half2_t p) { return (float)p.x + (float)p.y; }

// Sum over this lane's 32 K values of x * q * s, from 16 bytes of packed row
// (8 nibbles per dword), for activations whose odd pairs (m = 1, 3: slots 4q+1, 4q+3) are
// held divided by 16.  The nibbles of those pairs are then used in place as
// 1024 + 16u (one and-or, no shift): (x/16)(1024 + 16u) = 64x + xu, so the
// offset term is corr = 1032 * (sum of the even-pair x) + 1152 * (sum of the
// stored odd-pair x/16) and the result is s * (acc - corr).  Per lane (32 K
// values, inside one scale group) the offset cancels exactly while x/16 is an
// fp16 normal.
// Nibble masks in SGPRs and the fp16 exponent pattern in a VGPR, through
// asm the compiler cannot see into: (d & mask) | magic written as plain C
// then becomes one v_and_or_b32 (VOP3 takes no literal operands here, so with
// the constants visible the compiler emits a separate and and or), and the
// scheduler places it freely.
struct PairRegs {
  uint32_t m0, m4, magic;
};
__device__ __forceinline__ PairRegs pair_regs() {
  PairRegs r;
  asm("s_mov_b32 %0, 0xf000f" : "=s"(r.m0));
  asm("s_mov_b32 %0, 0xf000f0" : "=s"(r.m4));
  asm("v_mov_b32 %0, 0x64006400" : "=v"(r.magic));
  return r;
}

// kFused: each nibble pair as one v_and_or_b32 (and_or_sv, volatile);
// otherwise the same instruction from plain C over pair_regs(), which leaves
// the compiler free to schedule it (the gate/up kernels keep their register
// counts that way).
template <bool kFused>
__device__ __forceinline__ float dot32_split(const uint4 wq, const half2_t *xp, float corr, float s) {
  const PairRegs k = pair_regs();
  auto pair = [&](uint32_t d, uint32_t m) {
    return __builtin_bit_cast(half2_t, kFused ? and_or_sv(d, m, 0x64006400u)
                                              : ((d & (m == 0x000F000Fu ? k.m0 : k.m4)) | k.magic));
  };
  float acc = 0.0f;
  const uint32_t d[4] = {wq.x, wq.y, wq.z, wq.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t d8 = d[q] >> 8;
    acc = __builtin_amdgcn_fdot2(xp[4 * q], pair(d[q], 0x000F000Fu), acc, false);
    acc = __builtin_amdgcn_fdot2(xp[4 * q + 1], pair(d[q], 0x00F000F0u), acc, false);
    acc = __builtin_amdgcn_fdot2(xp[4 * q + 2], pair(d8, 0x000F000Fu), acc, false);
    acc = __builtin_amdgcn_fdot2(xp[4 * q + 3], pair(d8, 0x00F000F0u), acc, false);
  }
  return s * (acc - corr);
}

// dot32_split for the three weight formats (FMT: 0 symmetric 4-bit, 1
// asymmetric 4-bit, 2 symmetric 5-bit), from the even- and odd-pair sums se
// and so of the activations (so over the stored x/16) and the lane's side
// data `aux`: its group's zero point z (asymmetric) or the fifth-bit word of
// its 32 weights (5-bit, bit 4i + q for element i of dword q).  The offset
// term is (1024 + z) se + (1024 + 16 z) so with z = 8 for the symmetric
// 4-bit format; the 5-bit one puts the fifth bits into bit 4 (low pairs) and
// bit 8 (high pairs) of each fp16 pair and subtracts 1040 se + 1280 so.
template <bool kFused, int FMT>
__device__ __forceinline__ float dot32_fmt(const uint4 wq, const half2_t *xp, float se, float so, float s,
                                           uint32_t aux) {
  const PairRegs k = pair_regs();
  auto pair = [&](uint32_t d, uint32_t m) {
    return kFused ? and_or_sv(d, m, 0x64006400u) : ((d & (m == 0x000F000Fu ? k.m0 : k.m4)) | k.magic);
  };
  float acc = 0.0f;
  const uint32_t d[4] = {wq.x, wq.y, wq.z, wq.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t d8 = d[q] >> 8;
    uint32_t p0 = pair(d[q], 0x000F000Fu), p1 = pair(d[q], 0x00F000F0u);
    uint32_t p2 = pair(d8, 0x000F000Fu), p3 = pair(d8, 0x00F000F0u);
    if constexpr (FMT == 2) {
      const uint32_t t1 = aux << (4 - q), t2 = aux >> (4 + q);
      p0 |= t1 & 0x00100010u;
      p1 |= t1 & 0x01000100u;
      p2 |= t2 & 0x00100010u;
      p3 |= t2 & 0x01000100u;
    }
    acc = __builtin_amdgcn_fdot2(xp[4 * q], __builtin_bit_cast(half2_t, p0), acc, false);
    acc = __builtin_amdgcn_fdot2(xp[4 * q + 1], __builtin_bit_cast(half2_t, p1), acc, false);
    acc = __builtin_amdgcn_fdot2(xp[4 * q + 2], __builtin_bit_cast(half2_t, p2), acc, false);
    acc = __builtin_amdgcn_fdot2(xp[4 * q + 3], __builtin_bit_cast(half2_t, p3), acc, false);
  }
  float corr;
  if constexpr (FMT == 2) {
    corr = 1040.0f * se + 1280.0f * so;
  } else {
    const float z = FMT == 1 ? (float)aux : 8.0f;
    corr = (1024.0f + z) * se + (1024.0f + 16.0f * z) * so;
  }
  return s * (acc - corr);
}

// The side data of one lane's 32 weights (K from kk) of matrix row `row`
// (K elements per row, group g): its group's zero point (format 1) or its
// fifth-bit word (format 2); 0 for format 0.
template <int FMT>
__device__ __forceinline__ uint32_t gemv_aux(const uint8_t *x, size_t row, int K, int g, int kk) {
  if constexpr (FMT == 1) {
    const int grp = kk / g;
    return (x[row * (K / g / 2) + (grp >> 1)] >> (4 * (grp & 1))) & 15u;
  } else if constexpr (FMT == 2) {
    return reinterpret_cast<const uint32_t *>(x)[row * (K / 32) + kk / 32];
  }
  return 0u;
}

// Sum over each group of W consecutive lanes (W a power of two), in every
// lane of the group, with DPP moves inside 16-lane rows instead of LDS
// permutes; the whole wavefront must be active.
template <int W>
__device__ __forceinline__ float dpp_group_sum(float v) {
  if constexpr (W >= 2) v += dpp_f32<0xB1>(v);    // quad_perm [1,0,3,2]
  if constexpr (W >= 4) v += dpp_f32<0x4E>(v);    // quad_perm [2,3,0,1]
  if constexpr (W == 8) v += dpp_f32<0x141>(v);   // row_half_mirror: the other quad of the 8
  if constexpr (W >= 16) {
    v += dpp_f32<0x124>(v);                       // row_ror 4
    v += dpp_f32<0x128>(v);                       // row_ror 8
  }
  if constexpr (W == 32) v += __shfl_xor(v, 16, kWave);
  if constexpr (W == 64) {
    const int b = __float_as_int(v);
    v = (__int_as_float(__builtin_amdgcn_readlane(b, 0)) + __int_as_float(__builtin_amdgcn_readlane(b, 16))) +
        (__int_as_float(__builtin_amdgcn_readlane(b, 32)) + __int_as_float(__builtin_amdgcn_readlane(b, 48)));
  }
  return v;
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
