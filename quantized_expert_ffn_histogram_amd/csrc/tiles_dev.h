// Device-side steps of the grouped-GEMM path's preparation, shared by its
// prologue kernel and by the routing and grouping kernels of the layer call
// (which take them over there, one kernel boundary each).
#pragma once
#include "moe_internal.h"

namespace strata {
namespace {

// Tile list from the expert offsets, one workgroup of 1024 threads (E <= 1024).
// Expert e's rows split into count_e / 128 full tiles and, if a remainder is
// left, one partial tile of ceil(rem / 32) token blocks.  Tiles are listed by
// cost class (4 blocks, then 3, 2, 1), each class in expert order, so the
// list is sorted by cost for the scheduler; `by_expert` gets the same tiles
// in expert order.  Positions come from one scan of
// a packed 64-bit count: bits 0-30 hold the 4-block tiles, then three 11-bit
// fields the 3-, 2- and 1-block ones (at most one per expert, so < 2048).
__device__ __forceinline__ void plan_tiles(const int *__restrict__ offsets, int E, Tile *__restrict__ tiles,
                                           Tile *__restrict__ by_expert, int *__restrict__ meta,
                                           unsigned long long *part) {
  const int e = threadIdx.x;
  const int lo = e < E ? offsets[e] : 0;
  const int c = e < E ? offsets[e + 1] - lo : 0;
  const int full = c / kGemmRows, rem = c - full * kGemmRows;
  const int cls = (rem + 31) >> 5;  // blocks of the partial tile, 0 if none
  auto field = [](int cl) { return 31 + 11 * (3 - cl); };
  const unsigned long long mine = (unsigned long long)(full + (cls == 4)) |
                                  (cls >= 1 && cls <= 3 ? 1ull << field(cls) : 0ull);
  // Inclusive scan of the packed counts: within each wavefront by shuffles,
  // then the 16 wavefront totals through LDS (one barrier).
  const int lane = e & (kWave - 1), wv = e / kWave;
  unsigned long long incl = mine;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const unsigned long long t = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += t;
  }
  if (lane == kWave - 1) part[wv] = incl;
  __syncthreads();
  unsigned long long tot = 0;
#pragma unroll
  for (int w = 0; w < 1024 / kWave; ++w) {
    const unsigned long long pw = part[w];
    if (w < wv) incl += pw;
    tot += pw;
  }
  const unsigned long long ex = incl - mine;
  auto count = [](unsigned long long v, int cl) {
    return cl == 4 ? (int)(v & 0x7FFFFFFFull) : (int)((v >> (31 + 11 * (3 - cl))) & 0x7FFull);
  };
  const int pos4 = count(ex, 4);
  const int epos = pos4 + count(ex, 3) + count(ex, 2) + count(ex, 1);
  for (int i = 0; i < full; ++i) {
    const Tile t{e, lo + i * kGemmRows, kGemmRows, 0};
    tiles[pos4 + i] = t;
    by_expert[epos + i] = t;
  }
  if (cls > 0) {
    int pos = cls == 4 ? pos4 + full : count(ex, cls);
    for (int cl = 4; cl > cls; --cl) pos += count(tot, cl);
    const Tile t{e, lo + full * kGemmRows, rem, 0};
    tiles[pos] = t;
    by_expert[epos + full] = t;
  }
  if (e == 0) meta[0] = count(tot, 4) + count(tot, 3) + count(tot, 2) + count(tot, 1);
}

// x (bf16) to fp16 in the GEMM's fragment slot order, 8 elements per slot:
// slot i of xq holds the pairs (0,4) (1,5) (2,6) (3,7) of x's slot i, the
// order in which the dequantized weights pair their K values.  Exact for
// magnitudes in fp16's normal range (bf16 has fewer mantissa bits); smaller
// ones round toward zero to fp16 subnormals, larger ones saturate.
// Grid-stride over slots, part `part` of `parts`.
__device__ __forceinline__ void convert_x_slots(const uint4 *__restrict__ x, uint4 *__restrict__ xq, size_t n8,
                                                int part, int parts) {
  const size_t stride = (size_t)parts * blockDim.x;
  for (size_t i = part * (size_t)blockDim.x + threadIdx.x; i < n8; i += stride) {
    const uint4 v = x[i];
    auto lo = [](uint32_t d) { return __uint_as_float(d << 16); };
    auto hi = [](uint32_t d) { return __uint_as_float(d & 0xFFFF0000u); };
    uint4 o;
    o.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo(v.x), lo(v.z)));
    o.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(hi(v.x), hi(v.z)));
    o.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo(v.y), lo(v.w)));
    o.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(hi(v.y), hi(v.w)));
    xq[i] = o;
  }
}

}  // namespace
}  // namespace strata
