// Expert FFN for a few pairs per expert (decode and draft-verify batches):
// bandwidth-bound GEMV kernels that stream each selected expert's packed
// weights from HBM once, with the int4 dequantization fused into the dot
// products.
//
// Decode reads every active weight once per step, so its ceiling is memory
// bandwidth divided by the bytes read per step (lqnn.cn static review §4.1);
// each decode token is a fresh trip through the weights, with one token plus
// up to three drafts verified in one pass ("两天移植，预填充提速8倍：Strata引擎
// 实测" (kongchang.com), section "Strata快在哪：不是魔法，是物流").  Only the
// experts selected this step are touched: the work list holds one entry per
// (expert, up to kGemvRows grouped rows).
//
// Dot products: a dword of 8 nibbles gives four fp16 pairs (1024 + u_m,
// 1024 + u_{m+4}) with one shift and one and-or; v_dot2_f32_f16 accumulates
// x * (1024 + u) in fp32, and per lane (32 K values, inside one group since
// g >= 32) the exact identity  sum x*q*s = s * (sum x*(1024+u) - 1032 * sum x)
// removes the offset.  x is converted to fp16 pairs in the same slot order
// once per work item.
//
//   gemv_gateup: work item = (entry, 16 h columns); wavefront = 4 columns; for
//                each column the gate row and the up row are reduced across
//                the wavefront and lane 0 writes h = silu(g)*u (fp16).
//   gemv_down:   work item = 8 output rows of H for ALL entries (each expert's
//                down rows are read once overall).  Wavefront w takes entries
//                w, w+4, ...; per-token partial sums go to LDS in entry order and
//                the four wavefronts' slots are added in fixed order, so the
//                combined output is deterministic without atomics.
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

struct GemvArgs {
  const uint16_t *x;      // bf16 [T][H]
  const uint8_t *gate, *up, *down;
  const uint16_t *gate_s, *up_s, *down_s;
  int T, H, I, g, k;
  const int *perm;
  const float *topk_w;
  const Tile *tiles;
  const int *meta;
  uint16_t *h;            // fp16 [pairs][I]
  float *out;             // fused: [T][H]; else y [pairs][H]
  int fused;
};

// H <= 4096: a lane covers K values [32*lane + 2048*c, +32) for c < H/2048 (or the
// first H/32 lanes when H < 2048).
constexpr int kMaxChunks = kGemvMaxHidden / 2048;

__global__ __launch_bounds__(256) void gemv_gateup_kernel(GemvArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ntiles = a.meta[0];
  const int colsets = a.I / kGemvGateUpColsPerWG;
  const int item = blockIdx.x;
  if (item >= ntiles * colsets) return;
  const int entry = item / colsets, cs = item - entry * colsets;
  const Tile tile = a.tiles[entry];
  const int e = tile.e, nrows = tile.rows;

  const int nchunks = (a.H + 2047) / 2048;
  const bool active = 32 * lane < min(a.H, 2048);

  // x fragments of the tile's tokens, fp16 pairs in slot order, and their sums.
  half2_t xp[kGemvRows][kMaxChunks][16];
  float xs[kGemvRows][kMaxChunks];
#pragma unroll
  for (int r = 0; r < kGemvRows; ++r)
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
      xs[r][c] = 0.0f;
      for (int i = 0; i < 16; ++i) xp[r][c][i] = half2_t{};
      if (r < nrows && c < nchunks && active) {
        const int t = a.perm[tile.row0 + r] / a.k;
        const uint4 *src = reinterpret_cast<const uint4 *>(a.x + (size_t)t * a.H + 2048 * c + 32 * lane);
#pragma unroll
        for (int q = 0; q < 4; ++q) bf16x8_pairs(src[q], &xp[r][c][4 * q]);
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) s += pair_sum(xp[r][c][i]);
        xs[r][c] = s;
      }
    }

  const int kb = a.H / 2, ng = a.H / a.g;
#pragma unroll 1
  for (int cc = 0; cc < kGemvGateUpColsPerWG / 4; ++cc) {
    const int n = cs * kGemvGateUpColsPerWG + wave * (kGemvGateUpColsPerWG / 4) + cc;
    float gs[kGemvRows], us[kGemvRows];
#pragma unroll
    for (int r = 0; r < kGemvRows; ++r) gs[r] = us[r] = 0.0f;
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
      if (c < nchunks && active) {
        const size_t row = (size_t)e * a.I + n;
        const int kk = 2048 * c + 32 * lane;
        const uint4 wg = *reinterpret_cast<const uint4 *>(a.gate + row * kb + kk / 2);
        const uint4 wu = *reinterpret_cast<const uint4 *>(a.up + row * kb + kk / 2);
        const float sg = (float)__builtin_bit_cast(_Float16, a.gate_s[row * ng + kk / a.g]);
        const float su = (float)__builtin_bit_cast(_Float16, a.up_s[row * ng + kk / a.g]);
#pragma unroll
        for (int r = 0; r < kGemvRows; ++r) {
          if (r < nrows) {
            gs[r] += dot32(wg, xp[r][c], xs[r][c], sg);
            us[r] += dot32(wu, xp[r][c], xs[r][c], su);
          }
        }
      }
    }
#pragma unroll
    for (int r = 0; r < kGemvRows; ++r) {
      if (r < nrows) {
        const float gv = group_sum<64>(gs[r]);
        const float uv = group_sum<64>(us[r]);
        if (lane == 0) {
          const float hv = gv / (1.0f + __expf(-gv)) * uv;
          reinterpret_cast<_Float16 *>(a.h)[(size_t)(tile.row0 + r) * a.I + n] = (_Float16)hv;
        }
      }
    }
  }
}

template <int LPR>  // lanes per down row = I / 32
__global__ __launch_bounds__(256) void gemv_down_kernel(GemvArgs a) {
  constexpr int RPI = kWave / LPR;  // rows per wavefront instruction
  constexpr int ITER = (kGemvDownRowsPerWG + RPI - 1) / RPI;
  __shared__ float part[4][kGemvMaxTokens][kGemvDownRowsPerWG];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = lane % LPR, rsel = lane / LPR;
  const int nbase = blockIdx.x * kGemvDownRowsPerWG;
  const int ntiles = a.meta[0];

  if (a.fused)
    for (int i = tid; i < 4 * kGemvMaxTokens * kGemvDownRowsPerWG; i += 256) (&part[0][0][0])[i] = 0.0f;
  __syncthreads();

  const int kb = a.I / 2, ng = a.I / a.g;
  for (int entry = wave; entry < ntiles; entry += 4) {
    const Tile tile = a.tiles[entry];
    const int e = tile.e, nrows = tile.rows;
    half2_t hp[kGemvRows][16];
    float hs[kGemvRows], wt[kGemvRows];
    int tok[kGemvRows];
#pragma unroll
    for (int r = 0; r < kGemvRows; ++r) {
      hs[r] = 0.0f;
      wt[r] = 0.0f;
      tok[r] = 0;
      if (r < nrows) {
        const int p = a.perm[tile.row0 + r];
        tok[r] = p / a.k;
        if (a.fused) wt[r] = a.topk_w[p];
        const uint4 *src = reinterpret_cast<const uint4 *>(a.h + (size_t)(tile.row0 + r) * a.I + 32 * sub);
#pragma unroll
        for (int q = 0; q < 4; ++q) f16x8_pairs(src[q], &hp[r][4 * q]);
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) s += pair_sum(hp[r][i]);
        hs[r] = s;
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) hp[r][i] = half2_t{};
      }
    }
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      const int nl = it * RPI + rsel;  // local output row
      const bool rowok = nl < kGemvDownRowsPerWG;
      const int n = nbase + (rowok ? nl : 0);
      const size_t row = (size_t)e * a.H + n;
      const uint4 wq = *reinterpret_cast<const uint4 *>(a.down + row * kb + 16 * sub);
      const float sd = (float)__builtin_bit_cast(_Float16, a.down_s[row * ng + (32 * sub) / a.g]);
#pragma unroll
      for (int r = 0; r < kGemvRows; ++r) {
        if (r < nrows) {
          const float yv = group_sum<LPR>(dot32(wq, hp[r], hs[r], sd));
          if (sub == 0 && rowok) {
            if (a.fused)
              part[wave][tok[r]][nl] += wt[r] * yv;
            else
              a.out[(size_t)(tile.row0 + r) * a.H + n] = yv;
          }
        }
      }
    }
  }
  if (!a.fused) return;
  __syncthreads();
  for (int i = tid; i < a.T * kGemvDownRowsPerWG; i += 256) {
    const int t = i / kGemvDownRowsPerWG, nl = i - t * kGemvDownRowsPerWG;
    const float v = ((part[0][t][nl] + part[1][t][nl]) + part[2][t][nl]) + part[3][t][nl];
    a.out[(size_t)t * a.H + nbase + nl] = v;
  }
}

}  // namespace

bool gemv_supported(int T, int H, int I) {
  const bool pow2 = I >= 128 && I <= 2048 && (I & (I - 1)) == 0;
  return T <= kGemvMaxTokens && H <= kGemvMaxHidden && (H <= 2048 ? (H & (H - 1)) == 0 : H % 2048 == 0) && pow2;
}

hipError_t launch_ffn_gemv(const uint16_t *x, int T, int k, const FfnWeights &w, const int *offsets,
                           const int *perm, const float *topk_w, float *y_or_out,
                           const FfnWorkspace &ws, hipStream_t s) {
  const long long pairs = (long long)T * k;
  const long long tiles_upper = (pairs + kGemvRows - 1) / kGemvRows + std::min<long long>(w.E, pairs);
  hipError_t err = launch_plan(offsets, w.E, kGemvRows, ws.tiles, ws.meta, s);
  if (err != hipSuccess) return err;
  GemvArgs a{};
  a.x = x;
  a.gate = w.gate;
  a.up = w.up;
  a.down = w.down;
  a.gate_s = w.gate_s;
  a.up_s = w.up_s;
  a.down_s = w.down_s;
  a.T = T;
  a.H = w.H;
  a.I = w.I;
  a.g = w.g;
  a.k = k;
  a.perm = perm;
  a.topk_w = topk_w;
  a.tiles = ws.tiles;
  a.meta = ws.meta;
  a.h = ws.h;
  a.out = y_or_out;
  a.fused = topk_w != nullptr;
  {
    KernelTimer timer("gemv_gateup", s);
    gemv_gateup_kernel<<<(int)(tiles_upper * (w.I / kGemvGateUpColsPerWG)), 256, 0, s>>>(a);
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  const int grid = w.H / kGemvDownRowsPerWG;
  KernelTimer timer("gemv_down", s);
  switch (w.I / 32) {
    case 4: gemv_down_kernel<4><<<grid, 256, 0, s>>>(a); break;
    case 8: gemv_down_kernel<8><<<grid, 256, 0, s>>>(a); break;
    case 16: gemv_down_kernel<16><<<grid, 256, 0, s>>>(a); break;
    case 32: gemv_down_kernel<32><<<grid, 256, 0, s>>>(a); break;
    default: gemv_down_kernel<64><<<grid, 256, 0, s>>>(a); break;
  }
  return hipGetLastError();
}

}  // namespace strata
