// Grouped expert GEMMs with the int4 dequantization fused into the matmul
// (matrix-core path, for prefill chunks with many tokens per expert).
//
// 4-bit weights are dequantized inside the matmul kernel, never expanded to a
// full-precision copy first (lqnn.cn static review §1.2; kongchang.com
// hands-on, MMQ note: low-bit weight blocks are dequantized during the matrix
// product), and all tokens routed to an expert share one fetch of its weights
// ("两天移植，预填充提速8倍：Strata引擎实测", section "Strata快在哪：不是魔法，是
// 物流").  SwiGLU is fused into the gate/up kernel's epilogue (activation fused
// with the FFN projection: yfxerp.com static review §5.1).
//
// Work item: a tile of up to 128 grouped rows of one expert (from the plan)
// times a slice of weight rows ("features").  Workgroup = 4 wavefronts; each
// wavefront owns NB blocks of 32 features for all of the tile's tokens, so
// every weight element is fetched and dequantized by exactly one wavefront:
//   gate/up: wavefront w owns NB/2 gate blocks and the NB/2 up blocks of the
//            same h columns (silu(g)*u is local to the lane);
//   down:    wavefront w owns NB blocks of output features.
// NB = 2: two workgroups per CU (accumulators plus operands fit 256 VGPRs),
// 3-stage ring.  (NB = 4 tiles halve the LDS reads per MFMA but need the AGPR
// file and one workgroup per CU; on gfx950 they measured slower, since a
// single wavefront per SIMD cannot hide the dequant, LDS and barrier
// latencies.)  Matrix cores: v_mfma_f32_32x32x16_f16
// with the dequantized weights as the A operand and token rows as B, so each
// lane's accumulator holds runs of four consecutive features of one token.
//
// Dequant in registers: a dword holds 8 nibbles u_0..u_7 (even K low); the
// pair (u_m, u_{m+4}) goes into the mantissas of two fp16 values with one
// and-or: the low nibbles of each half-word give 1024 + u (minus 1032 is q
// exactly), the next nibbles give 1024 + 16u (times 1/16 minus 72 is q
// exactly, one fma); the upper byte pair needs one shift.  Times the fp16 group
// scale gives fp16(q*s) with a single rounding: 13 VALU ops per 8 weights.  Fragment slot e therefore holds K
// offset (e>>1) + 4*(e&1) of its 8-block; token rows are stored in the same
// slot order, so the contraction runs over the true K.
//
// Pipeline: every operand moves global -> LDS with direct-to-LDS loads
// (global_load_lds), kStages-1 K chunks ahead, one barrier per chunk.
// Scheduling: persistent workgroups; workgroups reach the 8 XCDs round-robin
// by block index, and each XCD gets a contiguous range of (tile, slice) items
// so the slices of one tile, which share its token rows, meet in one L2.
#include <type_traits>

#include "moe_internal.h"

namespace strata {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kXcds = 8;
constexpr int kKC = kGemmKChunk;            // K per pipelined chunk (64)
constexpr int kSegs = kKC / 8;              // 16-byte segments per token row per chunk
constexpr int kStageSegs = kGemmRows * kSegs;

constexpr int kWaves = 4;  // wavefronts per workgroup

template <int NB>
struct Cfg {
  static constexpr int kStages = 3;                    // LDS ring depth
  static constexpr int kWgPerCu = 2;
  static constexpr int kBRows = kWaves * NB * 32;      // weight rows per workgroup
  static constexpr int kHCols = kWaves * NB * 16;      // gate/up: h columns per workgroup
  static constexpr int kOutCols = kWaves * NB * 32;    // down: output features per workgroup
};

struct GemmArgs {
  const uint16_t *A;   // fp16 rows in fragment slot order: gate/up: x [T][K]; down: h [pairs][K]
  const uint8_t *B0;   // gate or down, packed [E][N][K/2]
  const uint16_t *S0;  // fp16 scales [E][N][K/g]
  const uint8_t *B1;   // up (gate/up only)
  const uint16_t *S1;
  int N, K, g;
  const int *perm;
  int k;
  const Tile *tiles;
  const int *meta;     // meta[0] = number of tiles
  void *C;             // gate/up: h fp16 [pairs][N] (slot order); down: fp16 y [pairs][N] in pair
                       // order (fused combine follows) or fp32 y [pairs][N] in grouped order
  int nslices;
  int fused;
};

struct RowTables {
  int src[kGemmRows];  // gate/up: token row of x; down: grouped row of h
  int dst[kGemmRows];  // down: output row (pair index p for the fp16 y, grouped row otherwise)
};

template <int NB>
struct Stage {
  uint4 a[kStageSegs];              // token rows [row][segment], XOR-swizzled (a_slot)
  uint4 b[2 * Cfg<NB>::kBRows];     // [weight row][lane half]: 16 bytes = 32 K values
  uint32_t s[2 * Cfg<NB>::kBRows];  // [weight row][lane half]: fp16 group scale in the low half
};

template <int NB>
struct Ring {
  Stage<NB> *st[Cfg<NB>::kStages];
};

// Direct-to-LDS loads take an LDS-address-space pointer; the cast makes the
// conversion from the generic pointer of a __shared__ object explicit.
typedef __attribute__((address_space(3))) void *lds_ptr_t;
__device__ __forceinline__ lds_ptr_t as_lds(void *p) { return (lds_ptr_t)p; }

// Wait until at most N vector-memory operations of this wavefront are
// outstanding (expcnt and lgkmcnt left unconstrained), N < 64.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | 0x0F70);
}

// Compiler-only memory barrier: keeps loads, direct-to-LDS issues and LDS
// reads on their side of the explicit waits and barriers.
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// (a & m) | o as one v_and_or_b32 (m wavefront-uniform in an SGPR); written
// out because the compiler otherwise emits a separate and + or with literals.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t o) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(m), "v"(o));
  return r;
}
__device__ __forceinline__ half8 dequant8(uint32_t d, half2_t s2, uint32_t mask, uint32_t magic) {
  const half2_t off = {(_Float16)1032.0f, (_Float16)1032.0f};
  const half2_t sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const half2_t off16 = {(_Float16)-72.0f, (_Float16)-72.0f};
  const uint32_t d8 = d >> 8;
  const uint32_t r0 = and_or(d, mask, magic);
  const uint32_t r1 = and_or(d, mask << 4, magic);
  const uint32_t r2 = and_or(d8, mask, magic);
  const uint32_t r3 = and_or(d8, mask << 4, magic);
  const half2_t h0 = (__builtin_bit_cast(half2_t, r0) - off) * s2;
  const half2_t h1 = __builtin_elementwise_fma(__builtin_bit_cast(half2_t, r1), sixteenth, off16) * s2;
  const half2_t h2 = (__builtin_bit_cast(half2_t, r2) - off) * s2;
  const half2_t h3 = __builtin_elementwise_fma(__builtin_bit_cast(half2_t, r3), sixteenth, off16) * s2;
  return half8{h0.x, h0.y, h1.x, h1.y, h2.x, h2.y, h3.x, h3.y};
}

__device__ __forceinline__ uint32_t dword_of(const uint4 v, int j) {
  switch (j & 3) {
    case 0: return v.x;
    case 1: return v.y;
    case 2: return v.z;
    default: return v.w;
  }
}

// LDS position (16-byte units) of logical segment c of tile row r: the XOR
// spreads the 8 rows read by one 8-lane group of a ds_read_b128 over all bank
// quads.
__device__ __forceinline__ int a_slot(int r, int c) { return r * kSegs + (c ^ (r & 7)); }

template <int NB>
__device__ __forceinline__ int brow_of(int wave, int nb, int col) { return (wave * NB + nb) * 32 + col; }

// One K chunk of MFMAs from one stage: NMB token blocks x NB feature blocks x 4 K-steps.
template <int NB, int NMB>
__device__ __forceinline__ void mma_chunk(floatx16 (&acc)[NMB][NB], const Stage<NB> &st, int wave, int col,
                                          int half) {
  const uint32_t mask = __builtin_amdgcn_readfirstlane(0x000F000Fu);
  const uint32_t magic = __builtin_amdgcn_readfirstlane(0x64006400u);
  uint4 bw[NB];
  half2_t s2[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int br = brow_of<NB>(wave, nb, col);
    bw[nb] = st.b[br * 2 + half];
    const _Float16 sv = __builtin_bit_cast(_Float16, (uint16_t)st.s[br * 2 + half]);
    s2[nb] = half2_t{sv, sv};
  }
  // Token fragments are read one K-step ahead of the MFMAs that use them.
  half8 af[2][NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) af[0][mb] = __builtin_bit_cast(half8, st.a[a_slot(mb * 32 + col, 4 * half)]);
#pragma unroll
  for (int j = 0; j < kKC / 16; ++j) {
    if (j + 1 < kKC / 16) {
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
        af[(j + 1) & 1][mb] = __builtin_bit_cast(half8, st.a[a_slot(mb * 32 + col, 4 * half + j + 1)]);
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const half8 bf = dequant8(dword_of(bw[nb], j), s2[nb], mask, magic);
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bf, af[j & 1][mb], acc[mb][nb], 0, 0, 0);
    }
  }
}

// First weight row (within its matrix) of block nb of wavefront `wave` in a slice.
template <int MODE, int NB>
__device__ __forceinline__ int weight_row0(int slice, int wave, int nb) {
  if (MODE == 0) {
    const int hb = nb % (NB / 2);  // gate blocks first, then the up blocks of the same columns
    return slice * Cfg<NB>::kHCols + (wave * (NB / 2) + hb) * 32;
  }
  return slice * Cfg<NB>::kOutCols + (wave * NB + nb) * 32;
}

// One work item: the tile's rows (NMB 32-row blocks, nrows valid) x this
// workgroup's slice of weight rows, over all of K.  Loads, kStages-1 chunks
// ahead, all direct-to-LDS:
//   * token rows (fp16 slot order): wavefront instruction i fills segments
//     [(4i + wave)*64, +64), i.e. 8 rows x 128 bytes, XOR-swizzled;
//   * packed weights: 32 rows x 32 bytes per instruction;
//   * scales: 32 rows x 2 halves per instruction (a 2-byte direct-to-LDS load
//     writes one zero-extended dword per lane).
// Per chunk: wait for this wavefront's loads of the chunk, one barrier (every
// wavefront's loads have landed and the oldest stage is free), issue chunk
// c+kStages-1 into it, then dequant + MFMAs.  Past the last chunk the issue
// repeats the last chunk (loads are never skipped), so every wait counts the
// same number of operations.
template <int MODE, int NB, int NMB>
__device__ __forceinline__ void gemm_tile(const GemmArgs &a, const Ring<NB> &R, const RowTables &rt, int e,
                                          int row0, int nrows, int slice) {
  constexpr int S_ = Cfg<NB>::kStages;
  // Token-row loads: 4*NMB instructions of 8 rows per stage, spread over the
  // wavefronts; when they do not divide evenly the surplus instructions
  // repeat earlier ones (same bytes to the same LDS place), so every
  // wavefront issues the same count.
  constexpr int kAInst = 4 * NMB, AI = (kAInst + kWaves - 1) / kWaves;
  constexpr int V = AI + 2 * NB;  // direct-to-LDS loads per stage per wavefront
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wavefront-uniform
  const int col = lane & 31, half = lane >> 5;
  const int nchunks = a.K / kKC;

  // Load addresses: a wavefront-uniform base plus a 32-bit lane offset (bytes).
  uint32_t aoff[AI];
  int aseg[AI];  // first LDS segment of each token-row instruction
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    aseg[i] = ((kWaves * i + wave) % kAInst) * 64;
    const int p = aseg[i] + lane;
    const int r = p >> 3, c = (p & 7) ^ (r & 7);
    aoff[i] = ((uint32_t)rt.src[r] * (uint32_t)a.K + 8 * c) * 2;
  }
  const int col2 = lane >> 1, hh = lane & 1;  // weight-row loads: row lane>>1 of a block, half lane&1
  // The last slice of a matrix whose rows the slice width does not divide
  // has wavefronts past the end: they load row 0 (in bounds), take part in
  // the loads and barriers, and store nothing.
  const bool wave_rows_valid = weight_row0<MODE, NB>(slice, wave, 0) < a.N;
  const char *bbase[NB];
  const char *sbase[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int n0 = wave_rows_valid ? weight_row0<MODE, NB>(slice, wave, nb) : 0;
    const bool up = MODE == 0 && nb >= NB / 2;
    const uint8_t *B = up ? a.B1 : a.B0;
    const uint16_t *Sc = up ? a.S1 : a.S0;
    bbase[nb] = reinterpret_cast<const char *>(B + ((size_t)e * a.N + n0) * (a.K / 2));
    sbase[nb] = reinterpret_cast<const char *>(Sc + ((size_t)e * a.N + n0) * (a.K / a.g));
  }
  const uint32_t boff = (uint32_t)col2 * (a.K / 2) + 16 * hh;
  const uint32_t soff = ((uint32_t)col2 * (a.K / a.g)) * 2;
  const int g_shift = 31 - __clz(a.g);  // g is a power of two
  const char *abase = reinterpret_cast<const char *>(a.A);

  auto issue = [&](Stage<NB> &st, int c) {
    const int kc = c * kKC;
    const char *ab = abase + 2 * kc;
#pragma unroll
    for (int i = 0; i < AI; ++i) __builtin_amdgcn_global_load_lds(ab + aoff[i], as_lds(&st.a[aseg[i]]), 16, 0, 0);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int base = brow_of<NB>(wave, nb, 0) * 2;
      __builtin_amdgcn_global_load_lds(bbase[nb] + kc / 2 + boff, as_lds(&st.b[base]), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(sbase[nb] + 2 * ((kc + 32 * hh) >> g_shift) + soff, as_lds(&st.s[base]), 2,
                                       0, 0);
    }
  };

  floatx16 acc[NMB][NB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = floatx16{};

  const int last = nchunks - 1;
  compiler_fence();
#pragma unroll
  for (int st = 0; st < S_ - 1; ++st) issue(*R.st[st], min(st, last));

  auto step = [&](auto stage_tag, int c) {
    constexpr int S = decltype(stage_tag)::value;
    if constexpr (S < S_) {
      compiler_fence();
      wait_vmcnt<(S_ - 2) * V>();    // this wavefront's loads of chunk c are done
      __builtin_amdgcn_s_barrier();  // ... and every other wavefront's; stage S-1 is free
      compiler_fence();
      issue(*R.st[(S + S_ - 1) % S_], min(c + S_ - 1, last));
      compiler_fence();
      if (c < nchunks) mma_chunk<NB, NMB>(acc, *R.st[S], wave, col, half);
    }
  };
  for (int c0 = 0; c0 < nchunks; c0 += S_) {
    step(std::integral_constant<int, 0>{}, c0);
    step(std::integral_constant<int, 1>{}, c0 + 1);
    step(std::integral_constant<int, 2>{}, c0 + 2);
    step(std::integral_constant<int, 3>{}, c0 + 3);
  }
  compiler_fence();
  wait_vmcnt<0>();  // no load of this tile may land in the next tile's stages
  compiler_fence();

  // Epilogue.  Accumulator element v of a lane: token row mb*32 + col of the
  // tile, feature 8*(v/4) + 4*half + v%4 of its 32-feature block.
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) {
    const int r = mb * 32 + col;
    if (MODE == 0) {
#pragma unroll
      for (int hb = 0; hb < NB / 2; ++hb) {
        // h = silu(g) * u, fp16.  Lanes l and l^32 hold the low and high four
        // features of each 8-feature group; after one exchange each lane owns
        // two whole groups and stores them in fragment slot order (16 bytes).
        uint32_t hp[4][2];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float hv[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float gv = acc[mb][hb][4 * i + q], uv = acc[mb][hb + NB / 2][4 * i + q];
            hv[q] = gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * uv;
          }
          hp[i][0] = __builtin_bit_cast(uint32_t, half2_t{(_Float16)hv[0], (_Float16)hv[1]});
          hp[i][1] = __builtin_bit_cast(uint32_t, half2_t{(_Float16)hv[2], (_Float16)hv[3]});
        }
        uint32_t snd[4], rcv[4];
        snd[0] = half ? hp[0][0] : hp[2][0];
        snd[1] = half ? hp[0][1] : hp[2][1];
        snd[2] = half ? hp[1][0] : hp[3][0];
        snd[3] = half ? hp[1][1] : hp[3][1];
#pragma unroll
        for (int x = 0; x < 4; ++x) rcv[x] = __shfl_xor(snd[x], 32, kWave);
        if (r < nrows && wave_rows_valid) {
          uint16_t *hout =
              static_cast<uint16_t *>(a.C) + (size_t)(row0 + r) * a.N + weight_row0<0, NB>(slice, wave, hb);
#pragma unroll
          for (int gi = 0; gi < 2; ++gi) {
            const int grp = 2 * half + gi;  // 8-feature group this lane stores
            const uint32_t lo0 = half ? rcv[2 * gi] : hp[grp][0], lo1 = half ? rcv[2 * gi + 1] : hp[grp][1];
            const uint32_t hi0 = half ? hp[grp][0] : rcv[2 * gi], hi1 = half ? hp[grp][1] : rcv[2 * gi + 1];
            uint4 o;
            o.x = __builtin_amdgcn_perm(hi0, lo0, 0x05040100u);
            o.y = __builtin_amdgcn_perm(hi0, lo0, 0x07060302u);
            o.z = __builtin_amdgcn_perm(hi1, lo1, 0x05040100u);
            o.w = __builtin_amdgcn_perm(hi1, lo1, 0x07060302u);
            *reinterpret_cast<uint4 *>(hout + 8 * grp) = o;
          }
        }
      }
    } else if (r < nrows && wave_rows_valid) {
      const size_t row = (size_t)rt.dst[r] * a.N;
      if (a.fused) {  // fp16 y rows in pair order, summed by the combine kernel
        uint16_t *yrow = static_cast<uint16_t *>(a.C) + row;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int n = weight_row0<1, NB>(slice, wave, nb) + 8 * i + 4 * half;
            uint2 o;
            o.x = __builtin_bit_cast(uint32_t, half2_t{(_Float16)acc[mb][nb][4 * i], (_Float16)acc[mb][nb][4 * i + 1]});
            o.y = __builtin_bit_cast(uint32_t,
                                     half2_t{(_Float16)acc[mb][nb][4 * i + 2], (_Float16)acc[mb][nb][4 * i + 3]});
            *reinterpret_cast<uint2 *>(yrow + n) = o;
          }
      } else {  // fp32 y rows in grouped order
        float *yrow = static_cast<float *>(a.C) + row;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int n = weight_row0<1, NB>(slice, wave, nb) + 8 * i + 4 * half;
            *reinterpret_cast<float4 *>(yrow + n) =
                float4{acc[mb][nb][4 * i], acc[mb][nb][4 * i + 1], acc[mb][nb][4 * i + 2], acc[mb][nb][4 * i + 3]};
          }
      }
    }
  }
}

template <int MODE, int NB>
__device__ __forceinline__ void gemm_persistent(const GemmArgs &a, const Ring<NB> &R, RowTables &rt) {
  const int tid = threadIdx.x;
  const int total = a.meta[0] * a.nslices;
  const int xcd = blockIdx.x % kXcds, lb = blockIdx.x / kXcds, per_xcd_wgs = gridDim.x / kXcds;
  const int base = total / kXcds, rem = total % kXcds;
  const int cnt = base + (xcd < rem ? 1 : 0);
  const int start = xcd * base + min(xcd, rem);

  for (int local = lb; local < cnt; local += per_xcd_wgs) {
    const int item = start + local;
    const int entry = item / a.nslices, slice = item - entry * a.nslices;
    const Tile tile = a.tiles[entry];
    const int nmb = (tile.rows + 31) >> 5;

    __syncthreads();  // previous work item is done with LDS and the row tables
    if (tid < kGemmRows) {
      const int r = tid < tile.rows ? tid : 0;  // padding rows repeat row 0 (results dropped)
      const int p = a.perm[tile.row0 + r];
      if (MODE == 0) {
        rt.src[tid] = p / a.k;
      } else {
        rt.src[tid] = tile.row0 + r;
        rt.dst[tid] = a.fused ? p : tile.row0 + r;
      }
    }
    __syncthreads();
    switch (nmb) {
      case 1: gemm_tile<MODE, NB, 1>(a, R, rt, tile.e, tile.row0, tile.rows, slice); break;
      case 2: gemm_tile<MODE, NB, 2>(a, R, rt, tile.e, tile.row0, tile.rows, slice); break;
      case 3: gemm_tile<MODE, NB, 3>(a, R, rt, tile.e, tile.row0, tile.rows, slice); break;
      default: gemm_tile<MODE, NB, 4>(a, R, rt, tile.e, tile.row0, tile.rows, slice); break;
    }
  }
}

// The ring stages are distinct LDS objects so the compiler tracks each
// stage's direct-to-LDS loads separately instead of waiting for all of them.
template <int MODE>  // 0: gate/up + silu*mul -> h;  1: down -> y
__global__ __launch_bounds__(64 * kWaves, 2) void moe_gemm_nb2(GemmArgs a) {
  __shared__ Stage<2> st0, st1, st2;
  __shared__ RowTables rt;
  const Ring<2> R{{&st0, &st1, &st2}};
  gemm_persistent<MODE, 2>(a, R, rt);
}

// Tile list from the expert offsets: expert e gets ceil(count_e / rows_per_tile)
// consecutive tiles; one workgroup of 1024 threads (E <= 1024).
__device__ __forceinline__ void plan_tiles(const int *__restrict__ offsets, int E, int rows_per_tile,
                                           Tile *__restrict__ tiles, int *__restrict__ meta, int *part) {
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

// Prologue of the GEMM path: block 0 builds the tile list; every block
// converts x (bf16) to fp16 in fragment slot order (grid-stride, 8 elements
// per thread).
__global__ __launch_bounds__(1024) void prep_kernel(const int *__restrict__ offsets, int E, Tile *__restrict__ tiles,
                                                    int *__restrict__ meta, const uint4 *__restrict__ x,
                                                    uint4 *__restrict__ xq, size_t n8) {
  __shared__ int part[1024];
  if (blockIdx.x == 0) plan_tiles(offsets, E, kGemmRows, tiles, meta, part);
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n8; i += stride) {
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

// Persistent grid: wg_per_cu workgroups per CU (256 CUs), whole XCD rounds.
int persistent_grid(long long work_upper, int wg_per_cu) {
  const long long cap = 256LL * wg_per_cu;
  long long g = work_upper < cap ? work_upper : cap;
  g = (g + kXcds - 1) / kXcds * kXcds;
  return (int)(g < kXcds ? kXcds : g);
}

template <int MODE>
hipError_t launch_gemm(GemmArgs args, long long tiles_upper, int matrix_rows, hipStream_t s) {
  const int width = MODE == 0 ? Cfg<2>::kHCols : Cfg<2>::kOutCols;
  args.nslices = (matrix_rows + width - 1) / width;
  moe_gemm_nb2<MODE><<<persistent_grid(tiles_upper * args.nslices, Cfg<2>::kWgPerCu), 64 * kWaves, 0, s>>>(args);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ffn_gemm(const uint16_t *x, int T, int k, const FfnWeights &w, const int *offsets,
                           const int *perm, const float *topk_w, float *y_or_out,
                           const FfnWorkspace &ws, hipStream_t s) {
  const long long pairs = (long long)T * k;
  const long long tiles_upper = (pairs + kGemmRows - 1) / kGemmRows + std::min<long long>(w.E, pairs);
  const bool fused = topk_w != nullptr;
  hipError_t err;
  {
    KernelTimer timer("ffn_prep", s);
    const size_t n8 = (size_t)T * w.H / 8;
    const int blocks = (int)std::max<size_t>(1, std::min<size_t>(1024, (n8 + 1023) / 1024));
    prep_kernel<<<blocks, 1024, 0, s>>>(offsets, w.E, ws.tiles, ws.meta, reinterpret_cast<const uint4 *>(x),
                                        reinterpret_cast<uint4 *>(ws.xq), n8);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }

  GemmArgs g{};
  g.A = ws.xq;
  g.B0 = w.gate;
  g.S0 = w.gate_s;
  g.B1 = w.up;
  g.S1 = w.up_s;
  g.N = w.I;
  g.K = w.H;
  g.g = w.g;
  g.perm = perm;
  g.k = k;
  g.tiles = ws.tiles;
  g.meta = ws.meta;
  g.C = ws.h;
  g.fused = 0;
  {
    KernelTimer timer("gemm_gateup", s);
    if ((err = launch_gemm<0>(g, tiles_upper, w.I, s)) != hipSuccess) return err;
  }

  GemmArgs d = g;
  d.A = ws.h;
  d.B0 = w.down;
  d.S0 = w.down_s;
  d.B1 = nullptr;
  d.S1 = nullptr;
  d.N = w.H;
  d.K = w.I;
  d.C = fused ? static_cast<void *>(ws.y16) : static_cast<void *>(y_or_out);
  d.fused = fused ? 1 : 0;
  {
    KernelTimer timer("gemm_down", s);
    if ((err = launch_gemm<1>(d, tiles_upper, w.H, s)) != hipSuccess) return err;
  }
  if (fused) return launch_combine_pairs(ws.y16, topk_w, T, k, w.H, y_or_out, s);
  return hipSuccess;
}

}  // namespace strata
