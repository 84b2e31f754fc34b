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
// times a slice of weight rows ("features").  Each wavefront owns 2 blocks of
// 32 weight rows for all of the tile's tokens, so every weight element is
// fetched and dequantized by exactly one wavefront:
//   gate/up: wavefront w owns one gate block and the up block of the same h
//            columns (silu(g)*u is local to the lane);
//   down:    wavefront w owns two blocks of output features.
// 128 fp32 accumulators + operands fit 256 VGPRs: two wavefronts per SIMD.
// Matrix cores: v_mfma_f32_32x32x16_f16 with the dequantized weights as the A
// operand and token rows as B, so each lane's accumulator holds runs of four
// consecutive features of one token.
//
// Two pipelines, both moving every operand global -> LDS with direct-to-LDS
// loads (global_load_lds) ahead of the MFMAs:
//   * wide (the common shapes): 8 wavefronts, one workgroup per CU, K stages
//     of 128 in a 2-stage ring; weights are loaded 64 contiguous bytes per
//     row, and the fp16 scales once per 8 groups (16 bytes per row) into a
//     double-buffered window.  This halves the vector-memory instructions and
//     cache sectors per flop of the general pipeline, which is what bounds
//     these kernels (the per-CU load path, not HBM bandwidth).  Needs the
//     groups per row, K/g, to be a multiple of 8.  Every format: asymmetric
//     4-bit with a window of zero points beside the scales, 5-bit with its
//     fifth-bit words in a ring beside the stages (and 4-group scale windows
//     to make LDS room for them).
//   * general: 4 wavefronts, two workgroups per CU, K chunks of 64 in a
//     3-stage ring, one 2-byte scale load per row and chunk; every format,
//     for the shapes the wide pipeline does not take.
//
// Dequant in registers: a dword holds 8 nibbles u_0..u_7 (even K low); the
// pair (u_m, u_{m+4}) goes into the mantissas of two fp16 values with one
// and-or: the low nibbles of each half-word give 1024 + u (minus 1032 is q
// exactly), the next nibbles give 1024 + 16u (times 1/16 minus 72 is q
// exactly, one fma); the upper byte pair needs one shift.  Times the fp16 group
// scale gives fp16(q*s) with a single rounding: 13 VALU ops per 8 weights.
// Fragment slot e therefore holds K offset (e>>1) + 4*(e&1) of its 8-block;
// token rows are stored in the same slot order, so the contraction runs over
// the true K.
//
// Scheduling: persistent workgroups; workgroups reach the 8 XCDs round-robin
// by block index, and each XCD gets a contiguous range of (tile, slice) items
// so the slices of one tile, which share its token rows, meet in one L2.
#include <type_traits>

#include "moe_internal.h"
#include "tiles_dev.h"


namespace strata {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kXcds = 8;
constexpr int kNB = 2;  // 32-row weight blocks per wavefront

// Workgroup shape for W wavefronts.
template <int W>
struct Shape {
  static constexpr int kBRows = W * kNB * 32;    // weight rows per workgroup
  static constexpr int kHCols = W * kNB * 16;    // gate/up: h columns per workgroup
  static constexpr int kOutCols = W * kNB * 32;  // down: output features per workgroup
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
  const Tile *tiles;   // work list: sorted by cost (by_cost) or in expert order
  const int *meta;     // meta[0] = number of tiles
  int by_cost;
  void *C;             // gate/up: h fp16 [pairs][N] (slot order); down: fp16 y [pairs][N] in pair
                       // order (fused combine follows) or fp32 y [pairs][N] in grouped order
  int a_rows;          // rows of A (T for gate/up, pairs for down)
  int nslices;         // weight-row slices per tile
  int spi;             // slices per work item (consecutive slices of one tile)
  int fused;
  // Weight side data of the other formats (general pipeline): zero points,
  // two per byte [E][N][K/g/2] (asymmetric 4-bit), or fifth-bit words
  // [E][N][K/32] (5-bit), for B0 and B1.
  const uint8_t *X0, *X1;
  int tiled;           // packed codes in 32-row x 128-K tiles (packed_offset), else row-major
};

// Weight formats (values of strata_weight_format).
constexpr int kFmtInt4 = 0, kFmtInt4Asym = 1, kFmtInt5 = 2;

struct RowTables {
  int src[kGemmRows];  // gate/up: token row of x; down: grouped row of h
  int dst[kGemmRows];  // down: output row (pair index p for the fp16 y, grouped row otherwise)
};

// Direct-to-LDS loads take an LDS-address-space pointer; the cast makes the
// conversion from the generic pointer of a __shared__ object explicit.
typedef __attribute__((address_space(3))) void *lds_ptr_t;
__device__ __forceinline__ lds_ptr_t as_lds(void *p) { return (lds_ptr_t)p; }
// LDS address `byte_off` bytes into object `p`, with the offset hidden from
// the optimizer until this point (see gemm_tile_wide: it keeps the compiler
// from holding every load destination in its own SGPR).
__device__ __forceinline__ lds_ptr_t lds_at(void *p, uint32_t byte_off) {
  return (lds_ptr_t)((__attribute__((address_space(3))) char *)as_lds(p) + byte_off);
}

// Raw buffer resource over `bytes` bytes at `base` (offsets past the end read
// zeros).  Direct-to-LDS loads through a buffer resource are plain vector-
// memory operations to the compiler's wait-count tracking, so LDS reads that
// follow them keep exact lgkmcnt waits; the global-address form is treated as
// possibly touching LDS through its address as well and turns every later
// LDS wait of the stage into a full one.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}

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

// dequant8 for the three weight formats: the low nibble of each half-word
// gives 1024 + u, the next nibble 1024 + 16u (as in dequant8); then
//   asymmetric 4-bit: minus (1024 + z) and (64 + z) for the group's zero
//     point z (ce, co), both exact in fp16;
//   5-bit: the fifth bits of the dword's 8 elements come from word hw (bit
//     4i + b for element i of the 32-element word's dword b) into bit 4 of
//     the low pairs and bit 8 of the high ones (one and-or each), then
//     minus 1040 and 80.
template <int FMT>
__device__ __forceinline__ half8 dequant8_fmt(uint32_t d, half2_t s2, uint32_t mask, uint32_t magic, half2_t ce,
                                              half2_t co, uint32_t hw, int b) {
  const half2_t sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const uint32_t d8 = d >> 8;
  uint32_t r0 = and_or(d, mask, magic);
  uint32_t r1 = and_or(d, mask << 4, magic);
  uint32_t r2 = and_or(d8, mask, magic);
  uint32_t r3 = and_or(d8, mask << 4, magic);
  if constexpr (FMT == kFmtInt5) {
    const uint32_t t1 = hw << (4 - b), t2 = hw >> (4 + b);
    r0 |= t1 & 0x00100010u;
    r1 |= t1 & 0x01000100u;
    r2 |= t2 & 0x00100010u;
    r3 |= t2 & 0x01000100u;
  }
  const half2_t h0 = (__builtin_bit_cast(half2_t, r0) + ce) * s2;
  const half2_t h1 = __builtin_elementwise_fma(__builtin_bit_cast(half2_t, r1), sixteenth, co) * s2;
  const half2_t h2 = (__builtin_bit_cast(half2_t, r2) + ce) * s2;
  const half2_t h3 = __builtin_elementwise_fma(__builtin_bit_cast(half2_t, r3), sixteenth, co) * s2;
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

// Workgroup row (0 .. W*64-1) of row `col` of block nb of wavefront `wave`.
__device__ __forceinline__ int brow_of(int wave, int nb, int col) { return (wave * kNB + nb) * 32 + col; }

// First weight row (within its matrix) of block nb of wavefront `wave` in a slice.
template <int MODE, int W>
__device__ __forceinline__ int weight_row0(int slice, int wave, int nb) {
  if (MODE == 0) {
    const int hb = nb % (kNB / 2);  // gate blocks first, then the up blocks of the same columns
    return slice * Shape<W>::kHCols + (wave * (kNB / 2) + hb) * 32;
  }
  return slice * Shape<W>::kOutCols + (wave * kNB + nb) * 32;
}

// Where a wavefront's weight rows and scales start (row 0 of the expert for
// wavefronts past the matrix end: in bounds, results not stored).
template <int MODE, int W>
__device__ __forceinline__ void weight_bases(const GemmArgs &a, int e, int slice, int wave, bool valid,
                                             const char *(&bbase)[kNB], const char *(&sbase)[kNB]) {
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    const int n0 = valid ? weight_row0<MODE, W>(slice, wave, nb) : 0;
    const bool up = MODE == 0 && nb >= kNB / 2;
    const uint8_t *B = up ? a.B1 : a.B0;
    const uint16_t *Sc = up ? a.S1 : a.S0;
    bbase[nb] = reinterpret_cast<const char *>(B + ((size_t)e * a.N + n0) * (a.K / 2));
    sbase[nb] = reinterpret_cast<const char *>(Sc + ((size_t)e * a.N + n0) * (a.K / a.g));
  }
}

// Dequant constants held in registers the compiler cannot see through: the
// nibble masks in SGPRs, the fp16 exponent pattern in a VGPR, so that each
// masked insert is one v_and_or_b32 written as plain C (which the scheduler
// can then place like any other VALU instruction).
struct DequantRegs {
  uint32_t mask, mask4, magic;
};
__device__ __forceinline__ DequantRegs dequant_regs() {
  DequantRegs r;
  asm("s_mov_b32 %0, 0xf000f" : "=s"(r.mask));
  asm("s_mov_b32 %0, 0xf000f0" : "=s"(r.mask4));
  asm("v_mov_b32 %0, 0x64006400" : "=v"(r.magic));
  return r;
}
// Same arithmetic as dequant8: q = (1024 + u) - 1032 for the low nibble of a
// half-word, q = (1024 + 16u) / 16 - 72 for the next one, both exact in fp16,
// then one multiply by the group scale.
__device__ __forceinline__ half8 dequant8_c(uint32_t d, half2_t s2, const DequantRegs &k) {
  const half2_t off = {(_Float16)1032.0f, (_Float16)1032.0f};
  const half2_t sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const half2_t off16 = {(_Float16)-72.0f, (_Float16)-72.0f};
  const uint32_t d8 = d >> 8;
  const uint32_t r0 = (d & k.mask) | k.magic;
  const uint32_t r1 = (d & k.mask4) | k.magic;
  const uint32_t r2 = (d8 & k.mask) | k.magic;
  const uint32_t r3 = (d8 & k.mask4) | k.magic;
  const half2_t h0 = (__builtin_bit_cast(half2_t, r0) - off) * s2;
  const half2_t h1 = __builtin_elementwise_fma(__builtin_bit_cast(half2_t, r1), sixteenth, off16) * s2;
  const half2_t h2 = (__builtin_bit_cast(half2_t, r2) - off) * s2;
  const half2_t h3 = __builtin_elementwise_fma(__builtin_bit_cast(half2_t, r3), sixteenth, off16) * s2;
  return half8{h0.x, h0.y, h1.x, h1.y, h2.x, h2.y, h3.x, h3.y};
}

// Piece q (0..3) of the dequantization of one packed dword for both weight
// blocks: fp16 pair q of the eight weights (see dequant8_c), for block 0 and
// block 1 side by side so that no two dependent packed operations are
// adjacent.  Symmetric 4-bit: s2 = (s, s).  Asymmetric 4-bit: s2 = (s, ce)
// with ce = -(1024 + z) for the group's zero point z, so q = u - z is
// (1024 + u) + ce for a low nibble and (1024 + 16u)/16 + (ce + 960) for the
// next one, both exact, then one multiply by s.
// 5-bit: the fifth bits of the dword's 8 weights come from the lane's word
// hw of its 32-K block (bit 4i + b for weight i of dword b), shifted into bit
// 4 of the low pairs and bit 8 of the high ones, then minus 1040 and 80.
template <int FMT>
__device__ __forceinline__ void dequant_piece(int q, const uint32_t (&d)[kNB], const half2_t (&s2)[kNB],
                                              const DequantRegs &k, uint32_t (&out)[kNB][4],
                                              const uint32_t (&hw)[kNB] = {}, int b = 0) {
  const half2_t off = {(_Float16)1032.0f, (_Float16)1032.0f};
  const half2_t sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const half2_t off16 = {(_Float16)-72.0f, (_Float16)-72.0f};
  const half2_t c960 = {(_Float16)960.0f, (_Float16)960.0f};
  uint32_t r[kNB];
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    const uint32_t src = q < 2 ? d[nb] : d[nb] >> 8;
    r[nb] = (src & ((q & 1) ? k.mask4 : k.mask)) | k.magic;
    if constexpr (FMT == kFmtInt5) {
      const uint32_t t = q < 2 ? hw[nb] << (4 - b) : hw[nb] >> (4 + b);
      r[nb] |= t & ((q & 1) ? 0x01000100u : 0x00100010u);
    }
  }
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    const half2_t v = __builtin_bit_cast(half2_t, r[nb]);
    if constexpr (FMT == kFmtInt5) {
      const half2_t sixteenth5 = {(_Float16)0.0625f, (_Float16)0.0625f};
      const half2_t o5 = {(_Float16)-1040.0f, (_Float16)-1040.0f};
      const half2_t o80 = {(_Float16)-80.0f, (_Float16)-80.0f};
      const half2_t qv = (q & 1) ? __builtin_elementwise_fma(v, sixteenth5, o80) : v + o5;
      out[nb][q] = __builtin_bit_cast(uint32_t, qv * s2[nb]);
    } else if constexpr (FMT == kFmtInt4) {
      const half2_t qv = (q & 1) ? __builtin_elementwise_fma(v, sixteenth, off16) : v - off;
      out[nb][q] = __builtin_bit_cast(uint32_t, qv * s2[nb]);
    } else {
      const half2_t sb = __builtin_shufflevector(s2[nb], s2[nb], 0, 0);
      const half2_t cb = __builtin_shufflevector(s2[nb], s2[nb], 1, 1);
      const half2_t qv = (q & 1) ? __builtin_elementwise_fma(v, sixteenth, cb + c960) : v + cb;
      out[nb][q] = __builtin_bit_cast(uint32_t, qv * sb);
    }
  }
}

// One 128-K stage (8 K-steps of 16) of MFMAs, software-pipelined by hand:
// during the MFMAs of K-step j the weights of K-step j+1 are dequantized (in
// four pieces) and each token block's fragment of K-step j+1 is read from LDS
// right after the last MFMA that uses the current one.  `bread(h, nb)` gives
// the packed weights of 64-K half h, block nb; `afrag(j, mb)` token block
// mb's fragment of K-step j; `pre(j)` runs at the start of K-step j.  Each
// token block's group (two MFMAs, one fragment read, its dequant pieces) is
// closed by a scheduling barrier, so the order is the source order.
// `hread(h, nb)` (5-bit only) gives the fifth-bit word of 64-K half h,
// block nb for this lane's 32 K values.
template <int NMB, int FMT, typename BRead, typename AFrag, typename Pre, typename HRead>
__device__ __forceinline__ void mma_stage_pipelined(floatx16 (&acc)[NMB][kNB], BRead &&bread,
                                                    const half2_t (&s2)[2][kNB], AFrag &&afrag, Pre &&pre,
                                                    HRead &&hread) {
  const DequantRegs k = dequant_regs();
  uint4 bw[kNB];
  uint32_t hw[kNB] = {};
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) bw[nb] = bread(0, nb);
  if constexpr (FMT == kFmtInt5) {
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) hw[nb] = hread(0, nb);
  }
  half8 af[NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) af[mb] = afrag(0, mb);
  uint32_t bf[2][kNB][4];
  {
    uint32_t d[kNB];
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) d[nb] = dword_of(bw[nb], 0);
#pragma unroll
    for (int q = 0; q < 4; ++q) dequant_piece<FMT>(q, d, s2[0], k, bf[0], hw, 0);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    pre(j);
    const int cur = j & 1, jn = j + 1;
    uint32_t d[kNB];
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) d[nb] = dword_of(bw[nb], jn & 3);
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) {
        const half8 w = __builtin_bit_cast(half8, uint4{bf[cur][nb][0], bf[cur][nb][1], bf[cur][nb][2], bf[cur][nb][3]});
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(w, af[mb], acc[mb][nb], 0, 0, 0);
      }
      if (j < 7) {
        af[mb] = afrag(jn, mb);
#pragma unroll
        for (int q = mb * 4 / NMB; q < (mb + 1) * 4 / NMB; ++q)
          dequant_piece<FMT>(q, d, s2[jn >> 2], k, bf[cur ^ 1], hw, jn & 3);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (j == 2) {  // half 0's packed weights are dead after K-step 3's dequant
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) bw[nb] = bread(1, nb);
      if constexpr (FMT == kFmtInt5) {
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) hw[nb] = hread(1, nb);
      }
    }
  }
}

// Four K-steps (64 K) of MFMAs (general pipeline): token fragments from
// `afrag(j, mb)`, weights from the packed dwords of bw (one per K-step) and
// the scales s2.
template <int NMB, int FMT, typename AFrag>
__device__ __forceinline__ void mma_k64(floatx16 (&acc)[NMB][kNB], const uint4 (&bw)[kNB],
                                        const half2_t (&s2)[kNB], const half2_t (&ce)[kNB], const half2_t (&co)[kNB],
                                        const uint32_t (&hw)[kNB], AFrag &&afrag) {
  const uint32_t mask = __builtin_amdgcn_readfirstlane(0x000F000Fu);
  const uint32_t magic = __builtin_amdgcn_readfirstlane(0x64006400u);
  // Token fragments are read one K-step ahead of the MFMAs that use them.
  half8 af[2][NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) af[0][mb] = afrag(0, mb);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (j + 1 < 4) {
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) af[(j + 1) & 1][mb] = afrag(j + 1, mb);
    }
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
      const half8 bf = FMT == kFmtInt4 ? dequant8(dword_of(bw[nb], j), s2[nb], mask, magic)
                                       : dequant8_fmt<FMT>(dword_of(bw[nb], j), s2[nb], mask, magic, ce[nb], co[nb],
                                                           hw[nb], j);
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bf, af[j & 1][mb], acc[mb][nb], 0, 0, 0);
    }
  }
}

// Epilogue.  Accumulator element v of a lane: token row mb*32 + col of the
// tile, feature 8*(v/4) + 4*half + v%4 of its 32-feature block.
template <int MODE, int W, int NMB>
__device__ __forceinline__ void epilogue(const GemmArgs &a, const RowTables &rt, const floatx16 (&acc)[NMB][kNB],
                                         int row0, int nrows, int slice, int wave, int col, int half, bool valid) {
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) {
    const int r = mb * 32 + col;
    if (MODE == 0) {
#pragma unroll
      for (int hb = 0; hb < kNB / 2; ++hb) {
        // h = silu(g) * u, fp16.  Lanes l and l^32 hold the low and high four
        // features of each 8-feature group; after one exchange each lane owns
        // two whole groups and stores them in fragment slot order (16 bytes).
        uint32_t hp[4][2];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float hv[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float gv = acc[mb][hb][4 * i + q], uv = acc[mb][hb + kNB / 2][4 * i + q];
            hv[q] = gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * uv;
          }
          hp[i][0] = __builtin_bit_cast(uint32_t, half2_t{(_Float16)hv[0], (_Float16)hv[1]});
          hp[i][1] = __builtin_bit_cast(uint32_t, half2_t{(_Float16)hv[2], (_Float16)hv[3]});
        }
        // Half-wave swaps (v_permlane32_swap): for gi = 0, 1 the lanes of
        // half 0 receive the high four features of group 2gi from half 1 and
        // give it the low four of group 2gi + 1, so afterwards every lane
        // holds both halves (lo: from half 0, hi: from half 1) of the group
        // it stores, 2 * gi + half: the two lanes of a row store 32
        // consecutive bytes with one instruction.
        uint32_t lo[2][2], hi[2][2];
#pragma unroll
        for (int gi = 0; gi < 2; ++gi)
#pragma unroll
          for (int d = 0; d < 2; ++d) {
            const auto sw = __builtin_amdgcn_permlane32_swap(hp[2 * gi][d], hp[2 * gi + 1][d], false, false);
            lo[gi][d] = sw[0];
            hi[gi][d] = sw[1];
          }
        if (r < nrows && valid) {
          uint16_t *hout =
              static_cast<uint16_t *>(a.C) + (size_t)(row0 + r) * a.N + weight_row0<0, W>(slice, wave, hb);
#pragma unroll
          for (int gi = 0; gi < 2; ++gi) {
            const int grp = 2 * gi + half;  // 8-feature group this lane stores
            const uint32_t lo0 = lo[gi][0], lo1 = lo[gi][1], hi0 = hi[gi][0], hi1 = hi[gi][1];
            uint4 o;
            o.x = __builtin_amdgcn_perm(hi0, lo0, 0x05040100u);
            o.y = __builtin_amdgcn_perm(hi0, lo0, 0x07060302u);
            o.z = __builtin_amdgcn_perm(hi1, lo1, 0x05040100u);
            o.w = __builtin_amdgcn_perm(hi1, lo1, 0x07060302u);
            *reinterpret_cast<uint4 *>(hout + 8 * grp) = o;
          }
        }
      }
    } else if (r < nrows && valid) {
      const size_t row = (size_t)rt.dst[r] * a.N;
      if (a.fused) {  // fp16 y rows in pair order, summed by the combine kernel
        // As for h: one exchange with lane l^32 gives each lane two whole
        // 8-feature groups per block, stored as 16 bytes each, the two lanes
        // of a row storing 32 consecutive bytes per instruction.
        uint16_t *yrow = static_cast<uint16_t *>(a.C) + row;
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) {
          uint32_t yp[4][2];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            yp[i][0] = __builtin_bit_cast(uint32_t, half2_t{(_Float16)acc[mb][nb][4 * i], (_Float16)acc[mb][nb][4 * i + 1]});
            yp[i][1] =
                __builtin_bit_cast(uint32_t, half2_t{(_Float16)acc[mb][nb][4 * i + 2], (_Float16)acc[mb][nb][4 * i + 3]});
          }
          // The same half-wave swaps as for h.
#pragma unroll
          for (int gi = 0; gi < 2; ++gi) {
            const int grp = 2 * gi + half;  // 8-feature group this lane stores
            const auto s0 = __builtin_amdgcn_permlane32_swap(yp[2 * gi][0], yp[2 * gi + 1][0], false, false);
            const auto s1 = __builtin_amdgcn_permlane32_swap(yp[2 * gi][1], yp[2 * gi + 1][1], false, false);
            uint4 o;
            o.x = s0[0];  // features 0-1 of the group (from the half-0 lane)
            o.y = s1[0];  // 2-3
            o.z = s0[1];  // 4-5 (from the half-1 lane)
            o.w = s1[1];  // 6-7
            *reinterpret_cast<uint4 *>(yrow + weight_row0<1, W>(slice, wave, nb) + 8 * grp) = o;
          }
        }
      } else {  // fp32 y rows in grouped order
        float *yrow = static_cast<float *>(a.C) + row;
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int n = weight_row0<1, W>(slice, wave, nb) + 8 * i + 4 * half;
            *reinterpret_cast<float4 *>(yrow + n) =
                float4{acc[mb][nb][4 * i], acc[mb][nb][4 * i + 1], acc[mb][nb][4 * i + 2], acc[mb][nb][4 * i + 3]};
          }
      }
    }
  }
}

// Persistent loop over work items; `run_tile(nmb, tile, slice0, nsl)` does
// one: slices slice0 .. slice0+nsl-1 (spi of them, fewer at the end) of one
// tile.  Workgroups are dispatched to the XCDs round-robin, so blockIdx % 8
// names the XCD; the items of one tile always run side by side in one XCD's
// L2.  by_cost: the list is sorted by cost (number of 32-row token blocks,
// largest first); tile j belongs to XCD j % 8 and the XCD's workgroups take
// its items round-robin in that order, so the cheap tiles fill the gaps of
// the last round (longest-first list scheduling).  Otherwise (expert order)
// each XCD takes a contiguous range of items, so the tiles of one expert
// share its weights in L2.
template <int MODE, typename RunTile>
__device__ __forceinline__ void gemm_persistent(const GemmArgs &a, RowTables &rt, RunTile &&run_tile) {
  const int tid = threadIdx.x;
  const int ntiles = a.meta[0];
  const int ipt = (a.nslices + a.spi - 1) / a.spi;  // items per tile
  const int xcd = blockIdx.x % kXcds, lb = blockIdx.x / kXcds, per_xcd_wgs = gridDim.x / kXcds;
  int cnt, start;
  if (a.by_cost) {
    cnt = (ntiles > xcd ? (ntiles - xcd + kXcds - 1) / kXcds : 0) * ipt;
    start = 0;
  } else {
    const int total = ntiles * ipt, base = total / kXcds, rem = total % kXcds;
    cnt = base + (xcd < rem ? 1 : 0);
    start = xcd * base + min(xcd, rem);
  }

  for (int q = lb; q < cnt; q += per_xcd_wgs) {
    int entry, part;
    if (a.by_cost) {
      const int lt = q / ipt;
      part = q - lt * ipt;
      entry = lt * kXcds + xcd;
    } else {
      const int item = start + q;
      entry = item / ipt;
      part = item - entry * ipt;
    }
    const int slice0 = part * a.spi, nsl = min(a.spi, a.nslices - slice0);
    const Tile tile = a.tiles[entry];

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
    run_tile((tile.rows + 31) >> 5, tile, slice0, nsl);
  }
}

template <typename F>
__device__ __forceinline__ void dispatch_nmb(int nmb, F &&f) {
  switch (nmb) {
    case 1: f(std::integral_constant<int, 1>{}); break;
    case 2: f(std::integral_constant<int, 2>{}); break;
    case 3: f(std::integral_constant<int, 3>{}); break;
    default: f(std::integral_constant<int, 4>{}); break;
  }
}

// =========================================================================
// Wide pipeline: 8 wavefronts, K stages of 128, 2-stage ring, scale windows.
// =========================================================================
constexpr int kWideW = 8;
constexpr int kKS = 128;  // K per stage

struct WideStage {
  uint4 a[kGemmRows * 16];             // token rows [row][16-byte segment], XOR-swizzled (wa_slot)
  uint4 b[Shape<kWideW>::kBRows * 4];  // weight rows [row][16-byte quarter], XOR-swizzled (wb_slot)
};
// Weight rows' fp16 scales of 8 consecutive groups (16 bytes per row); for
// the 5-bit format 4 groups (8 bytes per row, as two dwords: the first of
// every row of a wavefront's 64, then the second), which leaves LDS room for
// the fifth-bit words.
template <int FMT>
struct ScaleWindow {
  uint4 s[FMT == kFmtInt5 ? Shape<kWideW>::kBRows / 2 : Shape<kWideW>::kBRows];
};
// 5-bit: the fifth-bit words of a stage (4 per row, 16 bytes), one per ring
// slot; a placeholder otherwise.
template <int FMT>
struct HiStage {
  uint4 h[FMT == kFmtInt5 ? Shape<kWideW>::kBRows : 1];
};
// Asymmetric 4-bit: the zero points of the same 8 groups (4 bytes per row,
// group i of the window in bits 4i..4i+3); a placeholder otherwise.
template <int FMT>
struct ZeroWindow {
  uint32_t z[FMT == kFmtInt4Asym ? Shape<kWideW>::kBRows : 1];
};

// Segment c (0..15) of token row r: 16 consecutive rows read by a ds_read_b128
// lane group land on 16 different bank quads.
__device__ __forceinline__ int wa_slot(int r, int c) { return r * 16 + (c ^ (r & 15)); }
// Quarter q (0..3, 32 K values) of weight row br: 16 consecutive rows spread
// over all 64 banks.
__device__ __forceinline__ int wb_slot(int br, int q) { return br * 4 + (q ^ ((br >> 2) & 3)); }

// One work item on the wide pipeline.  Per stage (128 K) a wavefront issues:
//   * token rows: NMB instructions of 4 rows x 256 bytes (instruction wave+8i);
//   * packed weights: 2 per block, 16 rows x 64 bytes each;
//   * on the first stage of every 8-group window: one 16-byte scale load per
//     weight row of the wavefront (64 rows), into the window buffer of the
//     window's parity (asymmetric 4-bit: and one 4-byte load of the window's
//     zero points per row, into the zero window of the same parity).
// Step c: wait for this wavefront's loads, one barrier (every wavefront's
// loads of stage c landed, and everyone is done with stage c-1, whose buffer
// is next), read this stage's scales, then dequant + MFMAs, with the loads of
// stage c+1 issued one per K-step between the MFMA groups (a wavefront's
// load issue then overlaps the other wavefronts' MFMAs instead of all
// wavefronts issuing together after the barrier).
// One work item of the wide pipeline: slices slice0 .. slice0+nsl-1 of one
// tile.  The K stages of consecutive slices form one pipeline: while the last
// stage of a slice is computed the first stage of the next is already in
// flight, and the slice's epilogue runs while it lands.
template <int MODE, int NMB, int FMT>
__device__ __forceinline__ void gemm_tile_wide(const GemmArgs &a, WideStage &st0, WideStage &st1,
                                               ScaleWindow<FMT> &sw0, ScaleWindow<FMT> &sw1, ZeroWindow<FMT> &zw0,
                                               ZeroWindow<FMT> &zw1, HiStage<FMT> &hs0, HiStage<FMT> &hs1,
                                               const RowTables &rt, int e, int row0, int nrows, int slice0,
                                               int nsl) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wavefront-uniform
  const int col = lane & 31, half = lane >> 5;
  const int nst = a.K / kKS;  // K stages per slice
  // g is 32, 64 or 128: group and window indexes are shifts.
  const int lg = 31 - __builtin_clz(a.g);  // log2(g)
  constexpr bool k5 = FMT == kFmtInt5;
  constexpr int kWinG = k5 ? 4 : 8;        // groups per scale window
  const int lpw = lg - (k5 ? 5 : 4);       // log2(stages per scale window)
  const int ngr = a.K >> lg;               // groups per weight row (a multiple of 8, or 1, 2, 4)
  // Scale windows per slice.  Rows of fewer than 8 groups have one window
  // per slice whose 16-byte load also covers the next row's first scales
  // (unused); for the block's last row that part lies past the buffer
  // resource's range and reads as zero.  (The 5-bit format takes the wide
  // pipeline only with K/g a multiple of 8.)
  const int nwin = ngr >= 8 ? ngr / kWinG : 1;

  uint32_t aoff[NMB];
#pragma unroll
  for (int i = 0; i < NMB; ++i) {
    const int p = (wave + kWideW * i) * 64 + lane;
    const int r = p >> 4, c = (p & 15) ^ (r & 15);
    aoff[i] = ((uint32_t)rt.src[r] * (uint32_t)a.K + 8 * c) * 2;
  }
  // Weight rows: row rr of a 32-row block, 16-byte quarter (swizzled) of the
  // stage's 64 bytes; consecutive stages are 64 bytes apart in a row-major
  // row, 2 KB apart (one tile) in the tiled layout.
  uint32_t boff[2];
  const uint32_t b_row = a.tiled ? 64u : (uint32_t)(a.K / 2);
  const uint32_t b_stage = a.tiled ? 2048u : (uint32_t)(kKS / 2);
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int rr = 16 * t + (lane >> 2);
    boff[t] = (uint32_t)rr * b_row + 16 * ((lane & 3) ^ ((rr >> 2) & 3));
  }
  const __amdgpu_buffer_rsrc_t ra = buffer_rsrc(a.A, (uint32_t)a.a_rows * (uint32_t)a.K * 2u);

  // Load cursor: slice lsl, stage lc is the next stage whose loads are issued;
  // rb / rs are buffer resources over that slice's weight rows and scale rows
  // of this wavefront's two blocks (32 rows each).
  constexpr int kRes = kNB;
  constexpr bool kAsym = FMT == kFmtInt4Asym;
  int lsl = slice0, lc = 0;
  __amdgpu_buffer_rsrc_t rb[kRes], rs[kRes], rz[kAsym ? kRes : 1], rh[k5 ? kRes : 1];
  // This lane's scale row (and zero-point or fifth-bit row) in its block.
  const uint32_t soff = (uint32_t)col * ngr * 2;
  const uint32_t zoff = (uint32_t)col * (ngr / 2);
  const uint32_t hoff = (uint32_t)col * (uint32_t)(a.K / 32) * 4u;
  auto bases = [&](int sl) {
    const bool v = weight_row0<MODE, kWideW>(sl, wave, 0) < a.N;
    const char *bb[kNB];
    const char *sb[kNB];
    weight_bases<MODE, kWideW>(a, e, sl, wave, v, bb, sb);
#pragma unroll
    for (int r = 0; r < kRes; ++r) {
      rb[r] = buffer_rsrc(bb[r], 32u * (uint32_t)a.K / 2);
      rs[r] = buffer_rsrc(sb[r], 32u * (uint32_t)ngr * 2);
      if constexpr (kAsym) {
        const int n0 = v ? weight_row0<MODE, kWideW>(sl, wave, r) : 0;
        const uint8_t *X = MODE == 0 && r >= kNB / 2 ? a.X1 : a.X0;
        rz[r] = buffer_rsrc(X + ((size_t)e * a.N + n0) * (size_t)(ngr / 2), 32u * (uint32_t)(ngr / 2));
      }
      if constexpr (k5) {
        const int n0 = v ? weight_row0<MODE, kWideW>(sl, wave, r) : 0;
        const uint8_t *X = MODE == 0 && r >= kNB / 2 ? a.X1 : a.X0;
        const size_t rowb = (size_t)(a.K / 32) * 4;
        rh[r] = buffer_rsrc(X + ((size_t)e * a.N + n0) * rowb, 32u * (uint32_t)rowb);
      }
    }
  };
  bases(lsl);
  // Scale windows alternate between sw0 and sw1 in load order.
  auto window_odd = [&](int sl, int win) { return (((sl - slice0) * nwin + win) & 1) != 0; };

  // Per-wavefront LDS offsets of the load destinations (token rows and scale
  // windows: 1 KB per wavefront; weight rows: 4 KB), re-derived through an
  // empty asm once per stage so that each destination is one scalar add from
  // them instead of a loop-invariant register of its own.
  uint32_t lds_w1k = 0, lds_w4k = 0;
  auto refresh_lds_offsets = [&]() {
    lds_w1k = (uint32_t)wave * 1024u;
    lds_w4k = (uint32_t)wave * 4096u;
    asm volatile("" : "+s"(lds_w1k), "+s"(lds_w4k));
  };
  auto issue_a = [&](WideStage &st, int i) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, lds_at(st.a, lds_w1k + (uint32_t)(kWideW * i) * 1024u), 16,
                                             aoff[i] + 2u * (uint32_t)(lc * kKS), 0, 0, 0);
  };
  auto issue_b = [&](WideStage &st, int q) {
    const int nb = q >> 1, t = q & 1;
    const uint32_t so = (uint32_t)lc * b_stage;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb[nb], lds_at(st.b, lds_w4k + (uint32_t)(nb * 2048 + t * 1024)), 16,
                                             boff[t], so, 0, 0);
  };
  // Scale window of the cursor's stage, if it starts one: lanes 0-31 load the
  // rows of block 0, lanes 32-63 those of block 1 (16 bytes = 8 groups each).
  // Asymmetric 4-bit: the window's zero points likewise, 4 bytes per row
  // (the wide pipeline takes this format only when K/g is a multiple of 8,
  // so every row's window is a whole aligned dword).
  auto issue_s = [&]() {
    if ((lc & ((1 << lpw) - 1)) == 0) {
      const int win = lc >> lpw;
      const bool odd = window_odd(lsl, win);
      if constexpr (k5) {  // 8 bytes per row as two dword loads, 512 bytes per wavefront
        const lds_ptr_t dst = odd ? lds_at(sw1.s, lds_w1k >> 1) : lds_at(sw0.s, lds_w1k >> 1);
        const lds_ptr_t dst2 = odd ? lds_at(sw1.s, (lds_w1k >> 1) + 256u) : lds_at(sw0.s, (lds_w1k >> 1) + 256u);
        if (half == 0) {
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs[0], dst, 4, soff, 8u * win, 0, 0);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs[0], dst2, 4, soff, 8u * win + 4u, 0, 0);
        } else {
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs[1], dst, 4, soff, 8u * win, 0, 0);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs[1], dst2, 4, soff, 8u * win + 4u, 0, 0);
        }
      } else {
        const lds_ptr_t dst = odd ? lds_at(sw1.s, lds_w1k) : lds_at(sw0.s, lds_w1k);
        if (half == 0)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs[0], dst, 16, soff, 16u * win, 0, 0);
        else
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs[1], dst, 16, soff, 16u * win, 0, 0);
      }
      if constexpr (kAsym) {
        const uint32_t zw = lds_w1k >> 2;  // 256 bytes per wavefront
        const lds_ptr_t zdst = odd ? lds_at(zw1.z, zw) : lds_at(zw0.z, zw);
        if (half == 0)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rz[0], zdst, 4, zoff, 4u * win, 0, 0);
        else
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rz[kRes - 1], zdst, 4, zoff, 4u * win, 0, 0);
      }
    }
  };
  // The loads of the cursor's stage, spread over the 8 K-steps (kk) of the
  // stage computed meanwhile: the weight rows (from HBM, the longest latency)
  // all at the first K-step, so their latency has the whole stage to land,
  // and the token rows (mostly L2 hits) one per K-step after that.  kk is a
  // compile-time constant in every caller: no branch splits a K-step.
  // 5-bit: the stage's fifth-bit words (16 bytes per row: lanes 0-31 the rows
  // of block 0, 32-63 those of block 1) go with the weight rows into the
  // hi-word slot of the same ring position.
  auto issue_h = [&](HiStage<FMT> &hs) {
    if constexpr (k5) {
      if (half == 0)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rh[0], lds_at(hs.h, lds_w1k), 16, hoff, 16u * (uint32_t)lc, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rh[kRes - 1], lds_at(hs.h, lds_w1k), 16, hoff,
                                                 16u * (uint32_t)lc, 0, 0);
    }
  };
  auto issue_part = [&](WideStage &st, HiStage<FMT> &hs, int kk) {
    if (kk == 0) {
#pragma unroll
      for (int q = 0; q < 4; ++q) issue_b(st, q);
      issue_h(hs);
    } else if (kk <= NMB) {
      issue_a(st, kk - 1 < NMB ? kk - 1 : 0);
    }
  };
  auto advance_loads = [&]() {
    if (++lc == nst) {
      lc = 0;
      if (++lsl < slice0 + nsl) bases(lsl);
    }
  };

  floatx16 acc[NMB][kNB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) acc[mb][nb] = floatx16{};

  // Compute stage c of slice sl from `cur` while issuing the cursor's loads
  // into `nxt`.
  auto slice_epilogue = [&](int esl) {
    const bool valid = weight_row0<MODE, kWideW>(esl, wave, 0) < a.N;
    epilogue<MODE, kWideW, NMB>(a, rt, acc, row0, nrows, esl, wave, col, half, valid);
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) acc[mb][nb] = floatx16{};
  };
  // Compute stage c of slice sl from `cur`; with MORE (a compile-time flag:
  // this is not the item's last stage) issue the cursor's loads into `nxt`.
  auto step = [&](const WideStage &cur, WideStage &nxt, const HiStage<FMT> &hcur, HiStage<FMT> &hnxt, int sl, int c,
                  auto more_c) {
    constexpr bool MORE = decltype(more_c)::value;
    compiler_fence();
    wait_vmcnt<0>();               // this wavefront's loads of this stage are done
    __builtin_amdgcn_s_barrier();  // ... and everyone's; the other stage buffer is free
    compiler_fence();
    refresh_lds_offsets();
    // Scales of this stage's two 64-K halves (group of K offset kc + 32*half).
    const int win = c >> lpw;
    const bool odd = window_odd(sl, win);
    const ScaleWindow<FMT> &sw = odd ? sw1 : sw0;
    // Asymmetric 4-bit: (s, ce), ce = -(1024 + z) (fp16 bits 0xE400 | z).
    uint32_t zwin[kNB];
    if constexpr (kAsym) {
      const ZeroWindow<FMT> &zw = odd ? zw1 : zw0;
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) zwin[nb] = zw.z[brow_of(wave, nb, col)];
    }
    half2_t s2[2][kNB];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int grp = ((c * kKS + 64 * s + 32 * half) >> lg) - kWinG * win;
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) {
        uint16_t bits;
        if constexpr (k5)  // dword grp/2 of the row, half grp%2
          bits = reinterpret_cast<const uint16_t *>(
              reinterpret_cast<const uint32_t *>(sw.s) + wave * 128 + (grp >> 1) * 64 + nb * 32 + col)[grp & 1];
        else
          bits = reinterpret_cast<const uint16_t *>(&sw.s[brow_of(wave, nb, col)])[grp];
        if constexpr (kAsym) {
          const uint32_t ce = 0xE400u | ((zwin[nb] >> (4 * grp)) & 15u);
          s2[s][nb] = __builtin_bit_cast(half2_t, (uint32_t)bits | (ce << 16));
        } else {
          const _Float16 sv = __builtin_bit_cast(_Float16, bits);
          s2[s][nb] = half2_t{sv, sv};
        }
      }
    }
    compiler_fence();
    // The scale window of the cursor's stage, if it starts one (the buffer it
    // fills was last read two windows ago).
    if constexpr (MORE) issue_s();
    mma_stage_pipelined<NMB, FMT>(
        acc, [&](int h, int nb) { return cur.b[wb_slot(brow_of(wave, nb, col), 2 * h + half)]; }, s2,
        [&](int j, int mb) {
          return __builtin_bit_cast(half8, cur.a[wa_slot(mb * 32 + col, 8 * (j >> 2) + 4 * half + (j & 3))]);
        },
        [&](int j) {
          if constexpr (MORE) issue_part(nxt, hnxt, j);
          __builtin_amdgcn_sched_barrier(0);
        },
        [&](int h, int nb) -> uint32_t {
          if constexpr (k5) {
            const uint4 w4 = hcur.h[brow_of(wave, nb, col)];
            return dword_of(w4, 2 * h + half);
          }
          return 0u;
        });
    if constexpr (MORE) advance_loads();
  };
  // After stage c of slice sl: the slice's epilogue once its last stage is in.
  int sl = slice0, c = 0;
  auto finish = [&]() {
    if (++c < nst) return;
    slice_epilogue(sl);
    c = 0;
    ++sl;
  };

  compiler_fence();
  refresh_lds_offsets();
  issue_s();  // the first scale window
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) issue_part(st0, hs0, kk);
  advance_loads();
  const std::true_type more;
  const std::false_type last;
  const int total = nsl * nst;
  int gs = 0;
  for (; gs + 2 < total; gs += 2) {
    step(st0, st1, hs0, hs1, sl, c, more);
    finish();
    step(st1, st0, hs1, hs0, sl, c, more);
    finish();
  }
  const bool two = gs + 1 < total;
  if (two) {
    step(st0, st1, hs0, hs1, sl, c, more);
    finish();
  }
  step(two ? st1 : st0, st0, two ? hs1 : hs0, hs0, sl, c, last);
  finish();
  // The last step issued nothing: no load of this item is in flight.
}

// The ring stages and scale windows are distinct LDS objects so the compiler
// tracks each one's direct-to-LDS loads separately.
template <int MODE, int FMT>  // MODE 0: gate/up + silu*mul -> h;  1: down -> y
__global__ __launch_bounds__(64 * kWideW, 1) void moe_gemm_wide(GemmArgs a) {
  __shared__ WideStage st0, st1;
  __shared__ ScaleWindow<FMT> sw0, sw1;
  __shared__ ZeroWindow<FMT> zw0, zw1;
  __shared__ HiStage<FMT> hs0, hs1;
  __shared__ RowTables rt;
  gemm_persistent<MODE>(a, rt, [&](int nmb, const Tile &tile, int slice0, int nsl) {
    dispatch_nmb(nmb, [&](auto n) {
      gemm_tile_wide<MODE, decltype(n)::value, FMT>(a, st0, st1, sw0, sw1, zw0, zw1, hs0, hs1, rt, tile.e,
                                                    tile.row0, tile.rows, slice0, nsl);
    });
  });
}

// =========================================================================
// General pipeline: 4 wavefronts, K chunks of 64, 3-stage ring.
// =========================================================================
constexpr int kGenW = 4;
constexpr int kKC = kGemmKChunk;  // K per pipelined chunk (64)
constexpr int kGenStages = 3;

template <int FMT>
struct GenStage {
  uint4 a[kGemmRows * 8];                // token rows [row][segment], XOR-swizzled (ga_slot)
  uint4 b[2 * Shape<kGenW>::kBRows];     // [weight row][lane half]: 16 bytes = 32 K values
  uint32_t s[2 * Shape<kGenW>::kBRows];  // [weight row][lane half]: fp16 group scale in the low half
  // [weight row][lane half]: the group's zero-point byte (asymmetric) or
  // the fifth-bit word of the half's 32 K values (5-bit)
  uint32_t x[FMT == kFmtInt4 ? 1 : 2 * Shape<kGenW>::kBRows];
};
// Ring depth: 3 stages, except for the down kernel in the other formats
// (their stages carry the side data): 2 there, so that two workgroups fit a
// CU's LDS.  The gate/up kernel in those formats (K = H, a long K loop) keeps
// the deeper ring at one workgroup per CU: measured faster for the 5-bit
// format (486 vs 711 us at the 6144-token chunk), equal for the asymmetric
// one; the down kernel gains from the second workgroup (307 -> 237, 286 ->
// 221 us).
template <int MODE, int FMT>
constexpr int gen_stages() { return FMT == kFmtInt4 || MODE == 0 ? kGenStages : 2; }
template <int FMT>
struct GenRing {
  GenStage<FMT> *st[kGenStages];  // the first gen_stages() are used
};

// Segment c (0..7) of token row r: the 8 rows read by one 8-lane group of a
// ds_read_b128 hit distinct bank quads.
__device__ __forceinline__ int ga_slot(int r, int c) { return r * 8 + (c ^ (r & 7)); }

// One work item on the general pipeline.  Per chunk a wavefront issues:
//   * token rows (fp16 slot order): instruction i fills segments
//     [(4i + wave)*64, +64), i.e. 8 rows x 128 bytes;
//   * packed weights: 32 rows x 32 bytes per block;
//   * scales: 32 rows x 2 halves per block (a 2-byte direct-to-LDS load
//     writes one zero-extended dword per lane);
//   * other formats: per block one more direct-to-LDS load of the same
//     shape, the zero-point byte (1 byte) or the fifth-bit word (4 bytes).
// Step c: wait for this wavefront's loads of chunk c, one barrier (every
// wavefront's loads landed and the oldest stage is free), issue chunk c+2
// into it, then dequant + MFMAs.  Past the last chunk the issue repeats the
// last chunk (loads are never skipped), so every wait counts the same number
// of operations.
template <int MODE, int NMB, int FMT>
__device__ __forceinline__ void gemm_tile_general(const GemmArgs &a, const GenRing<FMT> &R, const RowTables &rt,
                                                  int e, int row0, int nrows, int slice) {
  constexpr int S_ = gen_stages<MODE, FMT>();
  constexpr int V = NMB + (FMT == kFmtInt4 ? 2 : 3) * kNB;  // direct-to-LDS loads per stage per wavefront
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wavefront-uniform
  const int col = lane & 31, half = lane >> 5;
  const int nchunks = a.K / kKC;

  // 64-bit row addresses: this pipeline also takes the shapes whose A
  // operand spans 4 GiB or more (the wide one's buffer offsets are 32-bit).
  const char *abase = reinterpret_cast<const char *>(a.A);
  const char *arow[NMB];
#pragma unroll
  for (int i = 0; i < NMB; ++i) {
    const int p = (kGenW * i + wave) * 64 + lane;
    const int r = p >> 3, c = (p & 7) ^ (r & 7);
    arow[i] = abase + ((size_t)rt.src[r] * (size_t)a.K + 8 * c) * 2;
  }
  const int col2 = lane >> 1, hh = lane & 1;  // weight-row loads: row lane>>1 of a block, half lane&1
  const bool valid = weight_row0<MODE, kGenW>(slice, wave, 0) < a.N;
  const char *bbase[kNB];
  const char *sbase[kNB];
  weight_bases<MODE, kGenW>(a, e, slice, wave, valid, bbase, sbase);
  // Weight rows: row col2 of a 32-row block, 16-byte half hh of the chunk's
  // 32 bytes (chunk c at byte 32c of a row-major row; in the tiled layout at
  // tile c/2, byte 32*(c%2) of the row's 64).
  const bool tiled = a.tiled != 0;
  const uint32_t boff = (uint32_t)col2 * (tiled ? 64u : (uint32_t)(a.K / 2)) + 16 * hh;
  const uint32_t soff = ((uint32_t)col2 * (a.K / a.g)) * 2;
  const int g_shift = 31 - __clz(a.g);  // g is a power of two
  // Side data of the other formats: the row's zero-point bytes or fifth-bit words.
  const char *xbase[kNB];
  uint32_t xoff = 0;
  if constexpr (FMT != kFmtInt4) {
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
      const int n0 = valid ? weight_row0<MODE, kGenW>(slice, wave, nb) : 0;
      const bool up = MODE == 0 && nb >= kNB / 2;
      const size_t rowbytes = FMT == kFmtInt4Asym ? (size_t)(a.K / a.g / 2) : (size_t)(a.K / 32) * 4;
      xbase[nb] = reinterpret_cast<const char *>(up ? a.X1 : a.X0) + ((size_t)e * a.N + n0) * rowbytes;
    }
    xoff = FMT == kFmtInt4Asym ? (uint32_t)col2 * (uint32_t)(a.K / a.g / 2) : (uint32_t)col2 * (uint32_t)(a.K / 32) * 4;
  }

  auto issue = [&](GenStage<FMT> &st, int c) {
    const int kc = c * kKC;
#pragma unroll
    for (int i = 0; i < NMB; ++i)
      __builtin_amdgcn_global_load_lds(arow[i] + 2 * kc, as_lds(&st.a[(kGenW * i + wave) * 64]), 16, 0, 0);
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
      const int base = brow_of(wave, nb, 0) * 2;
      const uint32_t kcb = tiled ? (uint32_t)(kc >> 7) * 2048u + (uint32_t)((kc >> 1) & 63) : (uint32_t)(kc >> 1);
      __builtin_amdgcn_global_load_lds(bbase[nb] + kcb + boff, as_lds(&st.b[base]), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(sbase[nb] + 2 * ((kc + 32 * hh) >> g_shift) + soff, as_lds(&st.s[base]), 2,
                                       0, 0);
      if constexpr (FMT == kFmtInt4Asym)
        __builtin_amdgcn_global_load_lds(xbase[nb] + (((kc + 32 * hh) >> g_shift) >> 1) + xoff, as_lds(&st.x[base]),
                                         1, 0, 0);
      else if constexpr (FMT == kFmtInt5)
        __builtin_amdgcn_global_load_lds(xbase[nb] + 4 * ((kc >> 5) + hh) + xoff, as_lds(&st.x[base]), 4, 0, 0);
    }
  };

  floatx16 acc[NMB][kNB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) acc[mb][nb] = floatx16{};

  const int last = nchunks - 1;
  compiler_fence();
#pragma unroll
  for (int st = 0; st < S_ - 1; ++st) issue(*R.st[st], min(st, last));

  auto step = [&](auto stage_tag, int c) {
    constexpr int S = decltype(stage_tag)::value;
    compiler_fence();
    wait_vmcnt<(S_ - 2) * V>();    // this wavefront's loads of chunk c are done
    __builtin_amdgcn_s_barrier();  // ... and every other wavefront's; stage S-1 is free
    compiler_fence();
    issue(*R.st[(S + S_ - 1) % S_], min(c + S_ - 1, last));
    compiler_fence();
    if (c < nchunks) {
      const GenStage<FMT> &st = *R.st[S];
      uint4 bw[kNB];
      half2_t s2[kNB], ce[kNB], co[kNB];
      uint32_t hw[kNB];
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) {
        const int br = brow_of(wave, nb, col);
        bw[nb] = st.b[br * 2 + half];
        const _Float16 sv = __builtin_bit_cast(_Float16, (uint16_t)st.s[br * 2 + half]);
        s2[nb] = half2_t{sv, sv};
        ce[nb] = half2_t{(_Float16)-1032.0f, (_Float16)-1032.0f};
        co[nb] = half2_t{(_Float16)-72.0f, (_Float16)-72.0f};
        hw[nb] = 0;
        if constexpr (FMT == kFmtInt4Asym) {
          // the zero point of this lane's group: nibble (group & 1) of the byte
          const int grp = (c * kKC + 32 * half) >> g_shift;
          const int z = (int)((st.x[br * 2 + half] >> (4 * (grp & 1))) & 15u);
          ce[nb] = half2_t{(_Float16)(-1024 - z), (_Float16)(-1024 - z)};
          co[nb] = half2_t{(_Float16)(-64 - z), (_Float16)(-64 - z)};
        } else if constexpr (FMT == kFmtInt5) {
          hw[nb] = st.x[br * 2 + half];
          ce[nb] = half2_t{(_Float16)-1040.0f, (_Float16)-1040.0f};
          co[nb] = half2_t{(_Float16)-80.0f, (_Float16)-80.0f};
        }
      }
      mma_k64<NMB, FMT>(acc, bw, s2, ce, co, hw, [&](int j, int mb) {
        return __builtin_bit_cast(half8, st.a[ga_slot(mb * 32 + col, 4 * half + j)]);
      });
    }
  };
  for (int c0 = 0; c0 < nchunks; c0 += S_) {
    step(std::integral_constant<int, 0>{}, c0);
    step(std::integral_constant<int, 1>{}, c0 + 1);
    if constexpr (S_ == 3) step(std::integral_constant<int, 2>{}, c0 + 2);
  }
  compiler_fence();
  wait_vmcnt<0>();  // no load of this tile may land in the next tile's stages
  compiler_fence();
  epilogue<MODE, kGenW, NMB>(a, rt, acc, row0, nrows, slice, wave, col, half, valid);
}

// Two workgroups per CU where the LDS allows it (see gen_stages).
template <int MODE, int FMT>
__global__ __launch_bounds__(64 * kGenW, 2) void moe_gemm_general(GemmArgs a) {
  __shared__ GenStage<FMT> st0, st1;
  __shared__ std::conditional_t<gen_stages<MODE, FMT>() == 3, GenStage<FMT>, char> st2;
  __shared__ RowTables rt;
  GenStage<FMT> *third = &st1;  // unused with a 2-stage ring
  if constexpr (gen_stages<MODE, FMT>() == 3) third = &st2;
  const GenRing<FMT> R{{&st0, &st1, third}};
  gemm_persistent<MODE>(a, rt, [&](int nmb, const Tile &tile, int slice0, int nsl) {
    dispatch_nmb(nmb, [&](auto n) {
      for (int sl = slice0; sl < slice0 + nsl; ++sl)
        gemm_tile_general<MODE, decltype(n)::value, FMT>(a, R, rt, tile.e, tile.row0, tile.rows, sl);
    });
  });
}

// Prologue of the GEMM path: block 0 builds the tile list; every block
// converts x (bf16) to fp16 in fragment slot order (grid-stride, 8 elements
// per thread).
__global__ __launch_bounds__(1024) void prep_kernel(const int *__restrict__ offsets, int E, Tile *__restrict__ tiles,
                                                    Tile *__restrict__ by_expert, int *__restrict__ meta,
                                                    const uint4 *__restrict__ x,
                                                    uint4 *__restrict__ xq, size_t n8) {
  __shared__ unsigned long long part[1024];
  if (blockIdx.x == 0) plan_tiles(offsets, E, tiles, by_expert, meta, part);
  convert_x_slots(x, xq, n8, blockIdx.x, gridDim.x);
}

// Persistent grid: wg_per_cu workgroups per CU (256 CUs), whole XCD rounds.
int persistent_grid(long long work_upper, int wg_per_cu) {
  const long long cap = 256LL * wg_per_cu;
  long long g = work_upper < cap ? work_upper : cap;
  g = (g + kXcds - 1) / kXcds * kXcds;
  return (int)(g < kXcds ? kXcds : g);
}

#ifndef STRATA_GEMM_WIDE
#define STRATA_GEMM_WIDE 1
#endif
#ifndef STRATA_WIDE_MIN_STAGES
#define STRATA_WIDE_MIN_STAGES 8
#endif

// The wide pipeline when the scale windows align with the rows (K/g a
// multiple of 8, or a whole row of fewer than 8 groups in one window), the
// general one otherwise.
template <int MODE>
hipError_t launch_gemm(GemmArgs args, long long tiles_upper, int matrix_rows, int fmt, hipStream_t s) {
  // The wide pipeline addresses A through a buffer resource: 32-bit offsets.
  // It takes the asymmetric and 5-bit formats when K/g is a multiple of 8
  // (whole zero-point and 4-group scale windows).
  const bool wide_fmt = fmt == kFmtInt4 || ((fmt == kFmtInt4Asym || fmt == kFmtInt5) && (args.K / args.g) % 8 == 0);
  const bool wide = STRATA_GEMM_WIDE && wide_fmt && args.K % kKS == 0 &&
                    ((args.K / args.g) % 8 == 0 || args.K / args.g < 8) &&
                    (long long)args.a_rows * args.K * 2 < (1LL << 32);
  if (wide) {
    const int width = MODE == 0 ? Shape<kWideW>::kHCols : Shape<kWideW>::kOutCols;
    args.nslices = (matrix_rows + width - 1) / width;
    // Items of fewer than 8 K stages pay the pipeline fill too often; join
    // consecutive slices of a tile until an item has 8 or more.
    const int nst = args.K / kKS;
    args.spi = std::max(1, std::min(args.nslices, (STRATA_WIDE_MIN_STAGES + nst - 1) / nst));
    const long long items = tiles_upper * ((args.nslices + args.spi - 1) / args.spi);
    if (fmt == kFmtInt4Asym)
      moe_gemm_wide<MODE, kFmtInt4Asym><<<persistent_grid(items, 1), 64 * kWideW, 0, s>>>(args);
    else if (fmt == kFmtInt5)
      moe_gemm_wide<MODE, kFmtInt5><<<persistent_grid(items, 1), 64 * kWideW, 0, s>>>(args);
    else
      moe_gemm_wide<MODE, kFmtInt4><<<persistent_grid(items, 1), 64 * kWideW, 0, s>>>(args);
  } else {
    const int width = MODE == 0 ? Shape<kGenW>::kHCols : Shape<kGenW>::kOutCols;
    args.nslices = (matrix_rows + width - 1) / width;
    args.spi = 1;
    const long long items = tiles_upper * args.nslices;
    if (fmt == kFmtInt4Asym)
      moe_gemm_general<MODE, kFmtInt4Asym><<<persistent_grid(items, MODE == 0 ? 1 : 2), 64 * kGenW, 0, s>>>(args);
    else if (fmt == kFmtInt5)
      moe_gemm_general<MODE, kFmtInt5><<<persistent_grid(items, MODE == 0 ? 1 : 2), 64 * kGenW, 0, s>>>(args);
    else
      moe_gemm_general<MODE, kFmtInt4><<<persistent_grid(items, 2), 64 * kGenW, 0, s>>>(args);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ffn_gemm(const uint16_t *x, int T, int k, const FfnWeights &w, const int *offsets,
                           const int *perm, const float *topk_w, float *y_or_out,
                           const FfnWorkspace &ws, hipStream_t s, bool prepared) {
  const long long pairs = (long long)T * k;
  const long long tiles_upper = (pairs + kGemmRows - 1) / kGemmRows + std::min<long long>(w.E, pairs);
  const bool fused = topk_w != nullptr;
  hipError_t err;
  if (!prepared) {
    KernelTimer timer("ffn_prep", s);
    const size_t n8 = (size_t)T * w.H / 8;
    const int blocks = (int)std::max<size_t>(1, std::min<size_t>(1024, (n8 + 1023) / 1024));
    prep_kernel<<<blocks, 1024, 0, s>>>(offsets, w.E, ws.tiles, ws.tiles + ws.tile_cap, ws.meta,
                                        reinterpret_cast<const uint4 *>(x), reinterpret_cast<uint4 *>(ws.xq), n8);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }

  GemmArgs g{};
  g.A = ws.xq;
  g.a_rows = T;
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
  g.by_cost = 1;
  g.meta = ws.meta;
  g.C = ws.h;
  g.fused = 0;
  g.X0 = w.gate_x;
  g.X1 = w.up_x;
  g.tiled = w.tiled;
  {
    KernelTimer timer("gemm_gateup", s);
    if ((err = launch_gemm<0>(g, tiles_upper, w.I, w.fmt, s)) != hipSuccess) return err;
  }

  GemmArgs d = g;
  d.A = ws.h;
  d.a_rows = (int)pairs;
  d.B0 = w.down;
  d.S0 = w.down_s;
  d.B1 = nullptr;
  d.S1 = nullptr;
  d.N = w.H;
  d.K = w.I;
  d.C = fused ? static_cast<void *>(ws.y16) : static_cast<void *>(y_or_out);
  d.fused = fused ? 1 : 0;
  d.X0 = w.down_x;
  d.X1 = nullptr;
  // The down GEMM walks the tiles in expert order: its fp16 y rows then
  // reach memory in an order the combine kernel reads measurably faster
  // (50 vs 57 us at T=6144, k=10, H=2048), and the sorted order gains it
  // nothing.
  d.tiles = ws.tiles + ws.tile_cap;
  d.by_cost = 0;
  {
    KernelTimer timer("gemm_down", s);
    if ((err = launch_gemm<1>(d, tiles_upper, w.H, w.fmt, s)) != hipSuccess) return err;
  }
  if (fused) return launch_combine_pairs(ws.y16, topk_w, T, k, w.H, y_or_out, s);
  return hipSuccess;
}

}  // namespace strata
