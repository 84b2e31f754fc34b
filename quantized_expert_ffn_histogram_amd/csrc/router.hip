// Router projection in front of the top-k routing: logits = x . W_r^T.
//
// Each layer's router scores every expert for every token before the top-k
// selection picks the few that run ("两天移植，预填充提速8倍：Strata引擎实测"
// (kongchang.com), section "Strata快在哪：不是魔法，是物流", MoE note: 512
// experts, about 10 active; the routing principle of the Strata design
// notes, 原理一).  The projection is a dense bf16 matmul [T][H] x [H][E] with
// fp32 accumulation; the selection that follows is the routing kernel's, on
// the fp32 logits written here.
//
// Workgroup: 128 tokens x 128 experts, 4 wavefronts; wavefront w owns the
// 64 experts 64 (w % 2).. and the 64 tokens 64 (w / 2).. of the tile (2 x 2
// blocks of v_mfma_f32_32x32x16_bf16, router rows as A, token rows as B).
// K advances in stages of 64 through a 4-slot LDS ring filled by
// direct-to-LDS loads issued three stages ahead; a wavefront reads the
// fragments of stage s+1 into registers while its MFMAs of stage s run, so
// LDS reads, MFMAs and the loads of later stages overlap.  Each 128-byte
// row of a stage is stored as 8 16-byte segments XOR-swizzled by row / 2:
// the 16 rows of a ds_read_b128 lane group then cover all 64 banks once.
// Every product of two bf16 values is exact in fp32; only the accumulation
// rounds.
#include "moe_internal.h"

namespace strata {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void *lds_ptr_t;

constexpr int kRT = 128;  // tokens per workgroup
constexpr int kRE = 128;  // experts per workgroup
constexpr int kRK = 64;   // K per stage (8 segments of 16 bytes)

struct RouterStage {
  uint4 x[kRT * 8];  // token rows, [row][segment], swizzled (rslot)
  uint4 w[kRE * 8];  // router rows, same layout
};

__device__ __forceinline__ int rslot(int r, int c) { return r * 8 + (c ^ ((r >> 1) & 7)); }

__device__ __forceinline__ lds_ptr_t lds_at(void *p, uint32_t off) {
  return (lds_ptr_t)((__attribute__((address_space(3))) char *)(lds_ptr_t)p + off);
}

// One stage's fragments of a wavefront: [k block j][32-row block q].
struct RouterFrags {
  bf16x8 a[kRK / 16][2], b[kRK / 16][2];
};

__global__ __launch_bounds__(256) void router_logits_kernel(const uint16_t *__restrict__ x,
                                                            const uint16_t *__restrict__ wr, int T, int H, int E,
                                                            float *__restrict__ logits) {
  __shared__ RouterStage st0, st1, st2, st3;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int t0 = blockIdx.x * kRT, e0 = blockIdx.y * kRE;
  const int eb = 64 * (wave & 1), tb = 64 * (wave >> 1);

  // Load assignment: LDS slot p = 256 i + tid (i < 4) of each array holds
  // row r = p / 8, physical segment p % 8, i.e. logical segment
  // (p % 8) ^ ((r / 2) % 8).  Rows past T or E load the last valid row
  // (their results are not stored).
  const __amdgpu_buffer_rsrc_t rx =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(x), 0, (int)((uint32_t)T * (uint32_t)H * 2u), 0x00020000);
  const __amdgpu_buffer_rsrc_t rw =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(wr), 0, (int)((uint32_t)E * (uint32_t)H * 2u), 0x00020000);
  uint32_t xoff[4], woff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = 256 * i + tid, r = p >> 3, c = (p & 7) ^ ((r >> 1) & 7);
    const int tr = min(t0 + r, T - 1), er = min(e0 + r, E - 1);
    xoff[i] = ((uint32_t)tr * (uint32_t)H + 8u * c) * 2u;
    woff[i] = ((uint32_t)er * (uint32_t)H + 8u * c) * 2u;
  }
  const int nst = H / kRK;
  // Loads of stage s; past the last stage the last one is loaded again into
  // a slot nothing reads, so that every wait below counts the same number of
  // operations.
  auto issue = [&](RouterStage &st, int s) {
    const uint32_t k0 = (uint32_t)min(s, nst - 1) * kRK * 2u;  // byte offset of the stage in a row
    const uint32_t wbase = (uint32_t)(tid >> 6) * 1024u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, lds_at(st.x, wbase + 4096u * i), 16, xoff[i] + k0, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, lds_at(st.w, wbase + 4096u * i), 16, woff[i] + k0, 0, 0, 0);
    }
  };
  auto read = [&](RouterFrags &f, const RouterStage &st) {
#pragma unroll
    for (int j = 0; j < kRK / 16; ++j)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        f.a[j][q] = __builtin_bit_cast(bf16x8, st.w[rslot(eb + 32 * q + col, 2 * j + half)]);
        f.b[j][q] = __builtin_bit_cast(bf16x8, st.x[rslot(tb + 32 * q + col, 2 * j + half)]);
      }
  };
  floatx16 acc[4];  // [2 * token block + expert block]
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) acc[mb] = floatx16{};
  auto mma = [&](const RouterFrags &f) {
#pragma unroll
    for (int j = 0; j < kRK / 16; ++j)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[j][mb & 1], f.b[j][mb >> 1], acc[mb], 0, 0, 0);
  };
  // Step s: this thread's loads of stage s+1 are done once at most the 8 of
  // stage s+2 are outstanding; after the barrier everyone's are, and every
  // wavefront has finished its MFMAs of stage s-1, whose fragments were the
  // last reads of slot (s-1) % 4: stage s+3 goes there.  Then the fragments
  // of stage s+1 are read and the MFMAs of stage s (fragments read in the
  // step before) are issued.  (A bare s_barrier: __syncthreads' fence would
  // wait for every load.)
  RouterFrags f0, f1;
  // The scheduling barriers keep each step's MFMAs between its s_barriers
  // (left free, the compiler moves them next to the reads they consume).
  auto step = [&](RouterStage &next, RouterStage &ahead, RouterFrags &fcur, RouterFrags &fnext, int s) {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    issue(ahead, s + 3);
    read(fnext, next);
    mma(fcur);
  };
  issue(st0, 0);
  issue(st1, 1);
  issue(st2, 2);
  asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  read(f0, st0);
  // Whole ring turns inside the loop and the remainder after it: a step
  // skipped inside the loop would reach the loop head with other loads in
  // flight, and the compiler would then wait for all of them there.
  int s = 0;
  for (; s + 4 <= nst; s += 4) {
    step(st1, st3, f0, f1, s);
    step(st2, st0, f1, f0, s + 1);
    step(st3, st1, f0, f1, s + 2);
    step(st0, st2, f1, f0, s + 3);
  }
  if (s < nst) step(st1, st3, f0, f1, s);
  if (s + 1 < nst) step(st2, st0, f1, f0, s + 1);
  if (s + 2 < nst) step(st3, st1, f0, f1, s + 2);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no load may land after the workgroup ends

  // Accumulator element v of block mb: token tb + 32 (mb / 2) + col, expert
  // eb + 32 (mb % 2) + 8 (v / 4) + 4 half + v % 4 of the tile.
  const bool vec = (E & 3) == 0;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const int t = t0 + tb + 32 * (mb >> 1) + col;
    if (t >= T) continue;
    float *row = logits + (size_t)t * E;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int e = e0 + eb + 32 * (mb & 1) + 8 * g + 4 * half;
      if (vec && e + 3 < E) {
        *reinterpret_cast<float4 *>(row + e) =
            float4{acc[mb][4 * g], acc[mb][4 * g + 1], acc[mb][4 * g + 2], acc[mb][4 * g + 3]};
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (e + q < E) row[e + q] = acc[mb][4 * g + q];
      }
    }
  }
}

}  // namespace

hipError_t launch_router_logits(const uint16_t *x, int T, int H, const uint16_t *w_router, int E, float *logits,
                                hipStream_t s) {
  const dim3 grid(ceil_div(T, kRT), ceil_div(E, kRE)), block(256);
  KernelTimer timer("router_logits", s);
  router_logits_kernel<<<grid, block, 0, s>>>(x, w_router, T, H, E, logits);
  return hipGetLastError();
}

}  // namespace strata
