// Grouped expert GEMMs with the int4 dequantization fused into the matmul
// (matrix-core path, for prefill chunks with many tokens per expert).
//
// The pages' point is that 4-bit weights must be dequantized inside the matmul
// kernel, not expanded to a full-precision copy before it (lqnn.cn static
// review §1.2; kongchang.com hands-on, MMQ note: blocks of low-bit weights are
// dequantized during the matrix product), and that larger batches per expert
// amortise each expert's weight fetch ("两天移植，预填充提速8倍：Strata引擎实测",
// section "Strata快在哪：不是魔法，是物流").  The SwiGLU activation is fused into
// the gate/up kernel's epilogue and the weighted combine into the down kernel's
// (activation fused with the FFN projection: yfxerp.com static review §5.1).
//
// Work unit: a tile of up to 128 grouped rows of one expert (a Tile from the
// plan kernel) times a slice of output columns.  Workgroup = 4 wavefronts;
// each wavefront owns 64 B-matrix rows (two 32-column MFMA blocks) across all
// of the tile's rows, so every weight element is fetched and dequantized by
// exactly one wavefront of the workgroup:
//   gate/up: wavefront w owns h columns [w*32, w*32+32) of the slice, i.e. the
//            gate rows and the up rows of those columns (silu(g)*u is local);
//   down:    wavefront w owns output columns [w*64, w*64+64) of the slice.
// A (token rows) is staged per K chunk of 128 through LDS as fp16; every
// wavefront reads all of it.  Matrix cores: v_mfma_f32_32x32x16_f16.
//
// Dequant in registers: a dword holds 8 nibbles u_0..u_7 (even K low); the
// pair (u_m, u_{m+4}) is moved into the mantissas of two fp16 1024.0 values
// with one shift and one and-or, minus 1032 gives q exactly, times the fp16
// group scale gives fp16(q*s) with a single rounding.  Operand slot e of a
// fragment therefore holds K offset (e>>1) + 4*(e&1) of its 8-block; A is
// written to LDS in the same order, so the contraction is over the true K.
//
// Tile scheduling: persistent workgroups.  Workgroups are dispatched to the 8
// XCDs round-robin by block index; each XCD gets a contiguous range of
// (tile, slice) work items so that the slices of one tile (which share its A
// rows) run on the same XCD and hit its L2.
#include "moe_internal.h"

namespace strata {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kXcds = 8;
constexpr int kMB = kGemmRows / 32;            // 32-row MFMA blocks per tile
constexpr int kLdsLd = kGemmKChunk + 8;        // fp16 per LDS row (pad breaks bank aliasing)

struct GemmArgs {
  const void *A;          // gate/up: x bf16 [T][K]; down: h fp16 [pairs][K]
  const uint8_t *B0;      // gate or down, packed [E][N][K/2]
  const uint16_t *S0;     // fp16 scales [E][N][K/g]
  const uint8_t *B1;      // up (gate/up only)
  const uint16_t *S1;
  int N, K, g;
  const int *perm;
  int k;
  const float *topk_w;    // down, fused: routing weight per pair
  const Tile *tiles;
  const int *meta;        // meta[0] = number of tiles
  void *C;                // gate/up: h fp16 [pairs][N]; down: out [T][N] or y [pairs][N] (fp32)
  int nslices;
  int fused;
};

__device__ __forceinline__ half8 dequant8(uint32_t d, half2_t s2) {
  const half2_t off = {(_Float16)1032.0f, (_Float16)1032.0f};
  const uint32_t r0 = (d & 0x000F000Fu) | 0x64006400u;
  const uint32_t r1 = ((d >> 4) & 0x000F000Fu) | 0x64006400u;
  const uint32_t r2 = ((d >> 8) & 0x000F000Fu) | 0x64006400u;
  const uint32_t r3 = ((d >> 12) & 0x000F000Fu) | 0x64006400u;
  const half2_t h0 = (__builtin_bit_cast(half2_t, r0) - off) * s2;
  const half2_t h1 = (__builtin_bit_cast(half2_t, r1) - off) * s2;
  const half2_t h2 = (__builtin_bit_cast(half2_t, r2) - off) * s2;
  const half2_t h3 = (__builtin_bit_cast(half2_t, r3) - off) * s2;
  return half8{h0.x, h0.y, h1.x, h1.y, h2.x, h2.y, h3.x, h3.y};
}

__device__ __forceinline__ uint32_t dword_of(const uint4 (&r)[2], int j) {
  const uint4 v = r[j >> 2];
  switch (j & 3) {
    case 0: return v.x;
    case 1: return v.y;
    case 2: return v.z;
    default: return v.w;
  }
}

// 8 bf16 (natural K order) -> 8 fp16 in fragment slot order (0,4,1,5,2,6,3,7).
__device__ __forceinline__ uint4 bf16x8_to_f16_slots(uint4 v) {
  auto lo = [](uint32_t d) { return __uint_as_float(d << 16); };
  auto hi = [](uint32_t d) { return __uint_as_float(d & 0xFFFF0000u); };
  uint4 o;
  o.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo(v.x), lo(v.z)));
  o.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(hi(v.x), hi(v.z)));
  o.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo(v.y), lo(v.w)));
  o.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(hi(v.y), hi(v.w)));
  return o;
}

// 8 fp16 (natural K order) -> fragment slot order (0,4,1,5,2,6,3,7).
__device__ __forceinline__ uint4 f16x8_to_slots(uint4 v) {
  uint4 o;
  o.x = __builtin_amdgcn_perm(v.z, v.x, 0x05040100u);
  o.y = __builtin_amdgcn_perm(v.z, v.x, 0x07060302u);
  o.z = __builtin_amdgcn_perm(v.w, v.y, 0x05040100u);
  o.w = __builtin_amdgcn_perm(v.w, v.y, 0x07060302u);
  return o;
}

template <int MODE>  // 0: gate/up + silu*mul -> h;  1: down + weighted combine
__global__ __launch_bounds__(256, 2) void moe_gemm_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) _Float16 As[kGemmRows * kLdsLd];
  __shared__ int rtok[kGemmRows];
  __shared__ float rwt[kGemmRows];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;

  const int total = a.meta[0] * a.nslices;
  const int xcd = blockIdx.x % kXcds, lb = blockIdx.x / kXcds, per_xcd_wgs = gridDim.x / kXcds;
  const int base = total / kXcds, rem = total % kXcds;
  const int cnt = base + (xcd < rem ? 1 : 0);
  const int start = xcd * base + min(xcd, rem);

  for (int local = lb; local < cnt; local += per_xcd_wgs) {
    const int L = start + local;
    const int entry = L / a.nslices, slice = L - entry * a.nslices;
    const Tile tile = a.tiles[entry];
    const int e = tile.e, row0 = tile.row0, nrows = tile.rows;
    const int nmb = (nrows + 31) >> 5;

    __syncthreads();  // previous work item finished with LDS
    if (tid < kGemmRows) {
      int tok = 0;
      float wt = 0.0f;
      if (tid < nrows) {
        const int p = a.perm[row0 + tid];
        tok = p / a.k;
        if (MODE == 1 && a.fused) wt = a.topk_w[p];
      }
      rtok[tid] = tok;
      rwt[tid] = wt;
    }

    const uint8_t *bp[2];
    const uint16_t *sp[2];
    int ncol[2];
    if (MODE == 0) {
      const int n = slice * kGateUpColsPerWG + wave * 32 + col;
      ncol[0] = ncol[1] = n;
      bp[0] = a.B0 + ((size_t)e * a.N + n) * (a.K / 2);
      bp[1] = a.B1 + ((size_t)e * a.N + n) * (a.K / 2);
      sp[0] = a.S0 + ((size_t)e * a.N + n) * (a.K / a.g);
      sp[1] = a.S1 + ((size_t)e * a.N + n) * (a.K / a.g);
    } else {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int n = slice * kDownColsPerWG + wave * 64 + nb * 32 + col;
        ncol[nb] = n;
        bp[nb] = a.B0 + ((size_t)e * a.N + n) * (a.K / 2);
        sp[nb] = a.S0 + ((size_t)e * a.N + n) * (a.K / a.g);
      }
    }

    floatx16 acc[kMB][2];
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = floatx16{};

    for (int kc = 0; kc < a.K; kc += kGemmKChunk) {
      // Weights: this lane's 64 K values [kc + 64*half, +64) of its row = 32 bytes.
      uint4 raw[2][2];
      half2_t sA[2], sB[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const uint4 *src = reinterpret_cast<const uint4 *>(bp[nb] + kc / 2 + half * 32);
        raw[nb][0] = src[0];
        raw[nb][1] = src[1];
        const int k0 = kc + 64 * half;
        const _Float16 s0 = __builtin_bit_cast(_Float16, sp[nb][k0 / a.g]);
        const _Float16 s1 = __builtin_bit_cast(_Float16, sp[nb][(k0 + 32) / a.g]);
        sA[nb] = half2_t{s0, s0};
        sB[nb] = half2_t{s1, s1};
      }

      __syncthreads();  // LDS free (previous chunk read) and row table visible
      // Stage A rows [0,128) x K [kc, kc+128) as fp16 in slot order.
#pragma unroll
      for (int i = 0; i < (kGemmRows * kGemmKChunk / 8) / 256; ++i) {
        const int seg = tid + 256 * i;
        const int r = seg >> 4, c8 = seg & 15;
        uint4 v = {0u, 0u, 0u, 0u};
        if (r < nrows) {
          if (MODE == 0) {
            const uint16_t *x = static_cast<const uint16_t *>(a.A);
            v = *reinterpret_cast<const uint4 *>(x + (size_t)rtok[r] * a.K + kc + 8 * c8);
            v = bf16x8_to_f16_slots(v);
          } else {
            const uint16_t *h = static_cast<const uint16_t *>(a.A);
            v = *reinterpret_cast<const uint4 *>(h + (size_t)(row0 + r) * a.K + kc + 8 * c8);
            v = f16x8_to_slots(v);
          }
        }
        *reinterpret_cast<uint4 *>(&As[r * kLdsLd + 8 * c8]) = v;
      }
      __syncthreads();

#pragma unroll
      for (int j = 0; j < kGemmKChunk / 16; ++j) {
        half8 bf[2];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) bf[nb] = dequant8(dword_of(raw[nb], j), j < 4 ? sA[nb] : sB[nb]);
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb) {
          if (mb < nmb) {
            const half8 af = *reinterpret_cast<const half8 *>(&As[(mb * 32 + col) * kLdsLd + 64 * half + 8 * j]);
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
              acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af, bf[nb], acc[mb][nb], 0, 0, 0);
          }
        }
      }
    }

    // Epilogue.  Accumulator element v of a lane: row 8*(v/4) + 4*half + v%4, column `col`.
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb) {
      if (mb >= nmb) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = mb * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
        if (r >= nrows) continue;
        if (MODE == 0) {
          const float gv = acc[mb][0][v], uv = acc[mb][1][v];
          const float hv = gv / (1.0f + __expf(-gv)) * uv;
          _Float16 *hout = static_cast<_Float16 *>(a.C);
          hout[(size_t)(row0 + r) * a.N + ncol[0]] = (_Float16)hv;
        } else {
          float *outp = static_cast<float *>(a.C);
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) {
            const float yv = acc[mb][nb][v];
            if (a.fused)
              unsafeAtomicAdd(outp + (size_t)rtok[r] * a.N + ncol[nb], rwt[r] * yv);
            else
              outp[(size_t)(row0 + r) * a.N + ncol[nb]] = yv;
          }
        }
      }
    }
  }
}

__global__ __launch_bounds__(1024) void plan_kernel(const int *__restrict__ offsets, int E,
                                                    int rows_per_tile, Tile *__restrict__ tiles,
                                                    int *__restrict__ meta) {
  __shared__ int part[1024];
  const int e = threadIdx.x;
  const int lo = e < E ? offsets[e] : 0;
  const int c = e < E ? offsets[e + 1] - lo : 0;
  const int nt = (c + rows_per_tile - 1) / rows_per_tile;
  part[e] = nt;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = e >= off ? part[e - off] : 0;
    __syncthreads();
    part[e] += v;
    __syncthreads();
  }
  const int first = part[e] - nt;
  for (int i = 0; i < nt; ++i) {
    Tile t;
    t.e = e;
    t.row0 = lo + i * rows_per_tile;
    t.rows = min(rows_per_tile, c - i * rows_per_tile);
    t.pad = 0;
    tiles[first + i] = t;
  }
  if (e == 1023) meta[0] = part[1023];
}

__global__ void zero_kernel(float4 *p, size_t n4) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n4; i += (size_t)gridDim.x * blockDim.x)
    p[i] = float4{0.f, 0.f, 0.f, 0.f};
}

// Persistent grid: at most two workgroups per CU (256 CUs), whole XCD rounds.
int persistent_grid(long long work_upper) {
  long long g = work_upper < 512 ? work_upper : 512;
  g = (g + kXcds - 1) / kXcds * kXcds;
  return (int)(g < kXcds ? kXcds : g);
}

}  // namespace

hipError_t launch_plan(const int *offsets, int E, int rows_per_tile, Tile *tiles, int *meta,
                       hipStream_t s) {
  KernelTimer timer("ffn_plan", s);
  plan_kernel<<<1, 1024, 0, s>>>(offsets, E, rows_per_tile, tiles, meta);
  return hipGetLastError();
}

hipError_t launch_zero(float *p, size_t n, hipStream_t s) {
  const size_t n4 = n / 4;
  const int blocks = (int)std::min<size_t>(2048, (n4 + 255) / 256);
  KernelTimer timer("zero_out", s);
  if (blocks > 0) zero_kernel<<<blocks, 256, 0, s>>>(reinterpret_cast<float4 *>(p), n4);
  return hipGetLastError();
}

hipError_t launch_ffn_gemm(const uint16_t *x, int T, int k, const FfnWeights &w, const int *offsets,
                           const int *perm, const float *topk_w, float *y_or_out,
                           const FfnWorkspace &ws, hipStream_t s) {
  const long long pairs = (long long)T * k;
  const long long tiles_upper = (pairs + kGemmRows - 1) / kGemmRows + std::min<long long>(w.E, pairs);
  hipError_t err = launch_plan(offsets, w.E, kGemmRows, ws.tiles, ws.meta, s);
  if (err != hipSuccess) return err;

  GemmArgs g{};
  g.A = x;
  g.B0 = w.gate;
  g.S0 = w.gate_s;
  g.B1 = w.up;
  g.S1 = w.up_s;
  g.N = w.I;
  g.K = w.H;
  g.g = w.g;
  g.perm = perm;
  g.k = k;
  g.topk_w = nullptr;
  g.tiles = ws.tiles;
  g.meta = ws.meta;
  g.C = ws.h;
  g.nslices = w.I / kGateUpColsPerWG;
  g.fused = 0;
  {
    KernelTimer timer("gemm_gateup", s);
    moe_gemm_kernel<0><<<persistent_grid(tiles_upper * g.nslices), 256, 0, s>>>(g);
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;

  const bool fused = topk_w != nullptr;
  if (fused && (err = launch_zero(y_or_out, (size_t)T * w.H, s)) != hipSuccess) return err;
  GemmArgs d = g;
  d.A = ws.h;
  d.B0 = w.down;
  d.S0 = w.down_s;
  d.B1 = nullptr;
  d.S1 = nullptr;
  d.N = w.H;
  d.K = w.I;
  d.topk_w = topk_w;
  d.C = y_or_out;
  d.nslices = w.H / kDownColsPerWG;
  d.fused = fused ? 1 : 0;
  {
    KernelTimer timer("gemm_down", s);
    moe_gemm_kernel<1><<<persistent_grid(tiles_upper * d.nslices), 256, 0, s>>>(d);
  }
  return hipGetLastError();
}

}  // namespace strata
