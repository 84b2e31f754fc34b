// 4-bit KV cache: per-head symmetric quantization of key / value vectors,
// and attention of decode queries over the cache rows an indexer selected,
// with the dequantization fused into the attention's reads.
//
// The cache of keys and values can be kept in 4 bits per element (the
// optional 4-bit KV cache of the release notes, "40天64个版本：Strata如何用发
// 版密度定义AI本地推理路线图", release 0.1.8), quantized per head and
// symmetrically (lqnn.cn static review, §3.1, the KV-cache branch), with the
// dequantization moved into the operator that reads the cache instead of a
// separate pass (yfxerp.com static review, §4.2).  The attention reads only
// the ~2000 cache rows the indexer picked for each query
// ("两天移植，预填充提速8倍：Strata引擎实测" (kongchang.com), section
// "Strata快在哪：不是魔法，是物流", attention paragraph).
//
// Cache layout: codes [L][Hkv][D/2] (offset-binary nibbles u = q + 8, even
// element in the low nibble) and one fp16 scale per (position, head)
// [L][Hkv]; a position's Hkv head vectors are contiguous, so a selected
// position is one contiguous Hkv * 64-byte read.
//
// kv_quantize: 16 lanes per (token, head) vector: max |x| by a DPP
//   reduction, s = fp16(max / 7), q = clamp(rint(x / s), -8, 7); the code
//   decision is that of the fp32 quotient rounded to nearest (taken from an
//   exact remainder, see the kernel).
// sparse attention, two kernels:
//   partial (grid: query token x chunk of 32 or 64 selected positions, 256
//     threads): scores of all query heads against the chunk's keys (each
//     thread a quarter of a head vector, quad reduction), the chunk's
//     softmax numerators, and the weighted sum of its values, which were
//     staged in LDS while the scores were computed; writes (max, sum,
//     unnormalized output) per head and chunk;
//   merge (grid: query token x head, one thread per element): combines the
//     chunks in order with the usual rescaling by exp(m_c - M) - so the
//     result does not depend on scheduling.
#include <type_traits>

#include "moe_internal.h"

namespace strata {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kKvD = 128;        // head_dim
// Selected positions per workgroup: 64, or 32 when 64 would leave fewer
// than 256 workgroups (a decode step of a few tokens: 4 tokens x 2048
// positions measured 16.5 us with 32 against 21.1 with 64; 16 tokens 31.6
// with 64 against 36.0 with 32).
constexpr int kAttnChunkMin = 32, kAttnChunkMax = 64;
int attn_chunk(int Tq, int n_sel) {
  return (long long)Tq * ((n_sel + kAttnChunkMax - 1) / kAttnChunkMax) >= 256 ? kAttnChunkMax : kAttnChunkMin;
}
constexpr int kPartStride = kKvD + 4;  // floats per (token, head, chunk) partial: output, max, sum, pad

__device__ __forceinline__ float bf16_lo(uint32_t d) { return __uint_as_float(d << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t d) { return __uint_as_float(d & 0xFFFF0000u); }

// Each group of 16 lanes quantizes one vector of D = 128 bf16 values (row
// t*Hkv + h): lane l of the group holds elements 8l .. 8l+7 (one 16-byte
// load) and writes their 8 codes as one 32-bit word; max |x| is a DPP
// reduction inside the 16-lane row.  A wavefront does 4 rows per round and
// kKvRounds rounds, all loads issued before the first reduction.  Rows whose
// slot lies outside [0, L) are skipped.  One launch can encode two tensors
// of the same tokens (keys and values): rows [0, rows1) come from the first,
// rows [rows1, rows) from the second.
constexpr int kKvRounds = 4;
constexpr int kKvRowsPerWave = 4 * kKvRounds;

struct KvQuantArgs {
  const uint16_t *x[2];  // bf16 [T][Hkv][D] each
  uint8_t *codes[2];     // [L][Hkv][D/2]
  uint16_t *scale[2];    // fp16 [L][Hkv]
  int rows1, rows;       // rows of the first tensor, rows of both
  int Hkv, L;
  const int *slots;      // [T], shared by both tensors
};

__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));   // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_f32<0x4E>(v));   // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_f32<0x124>(v));  // row_ror 4
  v = fmaxf(v, dpp_f32<0x128>(v));  // row_ror 8
  return v;
}

__global__ __launch_bounds__(256) void kv_quantize_kernel(KvQuantArgs a) {
  const int lane = threadIdx.x & 63, sub = lane & 15;
  const int wrow0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * kKvRowsPerWave + (lane >> 4);
  const int Hkv = a.Hkv;
  u32x4_t d[kKvRounds];
  int slot[kKvRounds];
#pragma unroll
  for (int r = 0; r < kKvRounds; ++r) {
    const int row = wrow0 + 4 * r;
    const int second = row >= a.rows1, rr = row - (second ? a.rows1 : 0);
    const uint16_t *x = second ? a.x[1] : a.x[0];
    d[r] = row < a.rows ? *reinterpret_cast<const u32x4_t *>(x + (size_t)rr * kKvD + 8 * sub) : u32x4_t{0, 0, 0, 0};
    slot[r] = row < a.rows ? a.slots[rr / Hkv] : -1;
  }
#pragma unroll
  for (int r = 0; r < kKvRounds; ++r) {
    const int row = wrow0 + 4 * r;
    float v[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_lo(d[r][i]);
      v[2 * i + 1] = bf16_hi(d[r][i]);
    }
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
    const float amax = row16_max(m);  // every lane of the row group reaches this
    if (slot[r] < 0 || slot[r] >= a.L) continue;  // also rows past the end
    const int second = row >= a.rows1, rr = row - (second ? a.rows1 : 0);
    const int h = rr % Hkv;
    const _Float16 s16 = (_Float16)(amax / 7.0f);
    const float sc = (float)s16;
    // q = rint(x / s) with the fp32 quotient rounded to nearest, without a
    // division per element: q0 = rint(x * (1/s)) is within one of it, the
    // remainder x - q0*s is exact (an fma; q0*s and x share a narrow range),
    // and comparing it with s/2 decides, ties to even.  The fp32 quotient
    // is a half-integer only when x/s is one exactly (x is bf16 and s fp16,
    // so any other x/s lies further from k + 1/2 than its rounding error),
    // so this equals rint of the IEEE quotient.
    const bool zero = !(sc > 0.0f) || sc == __builtin_huge_valf();  // x / s rounds to 0 (all-zero row, s = inf)
    const float rs = 1.0f / sc, hs = 0.5f * sc;
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float q0 = __builtin_rintf(v[i] * rs);
      const float e = __builtin_fmaf(-q0, sc, v[i]);
      int q = (int)q0;
      if (e > hs || (e == hs && (q & 1))) ++q;
      else if (e < -hs || (e == -hs && (q & 1))) --q;
      q = zero ? 0 : min(max(q, -8), 7);
      word |= (uint32_t)(q + 8) << (4 * i);
    }
    const size_t dst = (size_t)slot[r] * Hkv + h;
    reinterpret_cast<uint32_t *>((second ? a.codes[1] : a.codes[0]) + dst * (kKvD / 2))[sub] = word;
    if (sub == 0) (second ? a.scale[1] : a.scale[0])[dst] = __builtin_bit_cast(uint16_t, s16);
  }
}

struct AttnArgs {
  const uint16_t *q;        // bf16 [Tq][Hq][D]
  const uint8_t *kc, *vc;   // codes [L][Hkv][D/2]
  const uint16_t *ks, *vs;  // fp16 scales [L][Hkv]
  const int *sel;           // [Tq][n_sel] or null (positions 0 .. n_sel-1)
  int Tq, Hq, Hkv, L, n_sel, nchunks;
  float sm_scale;
  float *part;              // [Tq][Hq][nchunks][kPartStride]: output, max, sum
  float *out;               // fp32 [Tq][Hq][D]
};

// The 8 nibbles of one dword (elements 8j .. 8j+7 in order) as floats u in
// [0, 15]: two masks and one byte conversion per element.
__device__ __forceinline__ void nib8(uint32_t w, float *o) {
  const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
  // (float)((v >> 8k) & 0xFF) is one v_cvt_f32_ubyte<k>.
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    o[2 * k] = (float)((lo >> (8 * k)) & 0xFFu);
    o[2 * k + 1] = (float)((hi >> (8 * k)) & 0xFFu);
  }
}

template <int G, int C>  // query heads per KV head, positions per workgroup
__global__ __launch_bounds__(256) void attn_partial_kernel(AttnArgs a) {
  constexpr int D = kKvD;
  constexpr int kMaxRounds = (C + 7) / 8;  // score rounds at Hkv = 8 (8 positions per round)
  const int tid = threadIdx.x;
  const int t = blockIdx.x / a.nchunks, chunk = blockIdx.x - t * a.nchunks;
  const int i0 = chunk * C, cnt = min(C, a.n_sel - i0);
  const int Hkv = a.Hkv, Hq = a.Hq;

  __shared__ int pos_s[C];
  __shared__ float score[32][C];            // [query head][position]
  __shared__ u32x4_t vrow[C * 8 * (D / 32)];  // [position][Hkv][D/2 bytes], up to Hkv = 8
  __shared__ float vscale[C][8];
  __shared__ float wts[C][32];  // [position][query head]: e_p * s_p (value weights)
  __shared__ float wsumh[32];   // per query head: sum over the chunk of e_p * s_p

  if (tid < C) {
    const int i = i0 + min(tid, cnt - 1);  // past the end: repeat the last position (weight 0)
    pos_s[tid] = a.sel ? a.sel[(size_t)t * a.n_sel + i] : i;
  }
  __syncthreads();

  // Every load of the workgroup goes out before the first use: this thread's
  // key words of all rounds and its query slices first, the values after
  // them; loads complete in order, so the scores wait only for the keys and
  // queries while the values are still in flight.
  // Scores: thread (position pl, head g, quarter qd) of a round, 4 * Hkv
  // threads per position.
  const int tpp = 4 * Hkv, ppr = 256 / tpp;  // threads per position, positions per round
  const int rounds = (C + ppr - 1) / ppr;    // <= kMaxRounds
  const int pr = tid / tpp, rem = tid - pr * tpp, g = rem >> 2, qd = rem & 3;
  // The loads are unconditional, from clamped in-range indices (rounds past
  // `rounds` and units past the chunk are loaded and never used), so that
  // they form one straight run with no branch between them, and the fp16
  // scales stay raw bits until their first use: a conversion next to its
  // load would make every later load wait for it.
  u32x4_t kw[kMaxRounds];
  uint32_t ksb[kMaxRounds];
#pragma unroll
  for (int r = 0; r < kMaxRounds; ++r) {
    const int pl = min(r * ppr + pr, C - 1);
    const size_t row = (size_t)pos_s[pl] * Hkv + g;
    kw[r] = reinterpret_cast<const u32x4_t *>(a.kc + row * (D / 2))[qd];
    ksb[r] = a.ks[row];
  }
  // This thread's query slices, loaded here and converted below.
  u32x4_t qraw[G][4];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const u32x4_t *qp = reinterpret_cast<const u32x4_t *>(a.q + ((size_t)t * Hq + g * G + hh) * D + 32 * qd);
#pragma unroll
    for (int c = 0; c < 4; ++c) qraw[hh][c] = qp[c];
  }
  asm volatile("" ::: "memory");  // keeps the issue order: keys, queries, then values
  // ... then the chunk's value rows and scales (staged to LDS below).
  const int units = C * Hkv * 4;  // 16-byte units of value rows
  constexpr int kVRegs = (C * 8 * 4 + 255) / 256;  // 16-byte value units per thread, up to Hkv = 8
  u32x4_t vreg[kVRegs];
#pragma unroll
  for (int r = 0; r < kVRegs; ++r) {
    const int u = min(tid + 256 * r, units - 1);
    const int pl = u / (Hkv * 4), w = u - pl * (Hkv * 4);
    vreg[r] = reinterpret_cast<const u32x4_t *>(a.vc + (size_t)pos_s[pl] * Hkv * (D / 2))[w];
  }
  constexpr int kSRegs = (C * 8 + 255) / 256;  // value scales per thread, up to Hkv = 8
  uint32_t vsb[kSRegs];
#pragma unroll
  for (int r = 0; r < kSRegs; ++r) {
    const int u = min(tid + 256 * r, C * Hkv - 1);
    const int pl = u / Hkv, gv = u - pl * Hkv;
    vsb[r] = a.vs[(size_t)pos_s[pl] * Hkv + gv];
  }
  asm volatile("" ::: "memory");  // every load above is issued before the first use below
  // This thread's query slices (G heads x 32 values) and their sums (the
  // offset term: q . (u - 8) = q . u - 8 sum(q)).
  float qv[G][32], qsum[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    qsum[hh] = 0.0f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const u32x4_t v = qraw[hh][c];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        qv[hh][8 * c + 2 * i] = bf16_lo(v[i]);
        qv[hh][8 * c + 2 * i + 1] = bf16_hi(v[i]);
        qsum[hh] += qv[hh][8 * c + 2 * i] + qv[hh][8 * c + 2 * i + 1];
      }
    }
  }
#pragma unroll
  for (int r = 0; r < kMaxRounds; ++r) {
    if (r >= rounds) break;
    const int pl = r * ppr + pr;
    float uf[32];
#pragma unroll
    for (int c = 0; c < 4; ++c) nib8(kw[r][c], uf + 8 * c);
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      float acc = 0.0f;
#pragma unroll
      for (int i = 0; i < 32; ++i) acc = fmaf(qv[hh][i], uf[i], acc);
      acc = fmaf(-8.0f, qsum[hh], acc) * (float)__builtin_bit_cast(_Float16, (uint16_t)ksb[r]);
      acc += dpp_f32<0xB1>(acc);  // quad reduction over the four quarters
      acc += dpp_f32<0x4E>(acc);
      if (qd == 0 && pl < C) score[g * G + hh][pl] = pl < cnt ? acc * a.sm_scale : -INFINITY;
    }
  }
  // The staged values go to LDS.
#pragma unroll
  for (int r = 0; r < kVRegs; ++r)
    if (tid + 256 * r < units) vrow[tid + 256 * r] = vreg[r];
#pragma unroll
  for (int r = 0; r < kSRegs; ++r) {
    const int u = tid + 256 * r;
    if (u < C * Hkv) vscale[u / Hkv][u % Hkv] = (float)__builtin_bit_cast(_Float16, (uint16_t)vsb[r]);
  }
  __syncthreads();

  // Chunk softmax numerators: head h = tid / 8, 8 threads x C/8 positions.
  // Each writes its positions' value weights w_p = e_p * s_p (s_p the value
  // row's scale) and the head's (max, sum of e) go straight to the partial.
  float *const part_t = a.part + (size_t)t * Hq * a.nchunks * kPartStride;
  if (tid < Hq * 8) {
    const int h = tid >> 3, j = tid & 7, gk = h / G;
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < C / 8; ++i) m = fmaxf(m, score[h][j * (C / 8) + i]);
    m = fmaxf(m, dpp_f32<0xB1>(m));
    m = fmaxf(m, dpp_f32<0x4E>(m));
    m = fmaxf(m, dpp_f32<0x141>(m));  // the other quad of the 8 lanes
    float l = 0.0f, ws = 0.0f;
#pragma unroll
    for (int i = 0; i < C / 8; ++i) {
      const int pl = j * (C / 8) + i;
      const float e = __expf(score[h][pl] - m);
      const float w = e * vscale[pl][gk];
      wts[pl][h] = w;
      l += e;
      ws += w;
    }
    l += dpp_f32<0xB1>(l);
    l += dpp_f32<0x4E>(l);
    l += dpp_f32<0x141>(l);
    ws += dpp_f32<0xB1>(ws);
    ws += dpp_f32<0x4E>(ws);
    ws += dpp_f32<0x141>(ws);
    if (j == 0) {
      float *dst = part_t + ((size_t)h * a.nchunks + chunk) * kPartStride;
      dst[D] = m;
      dst[D + 1] = l;
      wsumh[h] = ws;
    }
  }
  __syncthreads();

  // Weighted sum of the values: thread (KV head gk, dims 4 dq .. 4 dq + 3)
  // for all G query heads of gk, so each value code is unpacked once:
  // o = sum_p w_p (u_p - 8) = sum_p w_p u_p - 8 sum_p w_p.
  if (tid < Hkv * 32) {
    const int gk = tid >> 5, dq = tid & 31;
    float o[G][4];
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int i = 0; i < 4; ++i) o[hh][i] = 0.0f;
    const uint8_t *vb = reinterpret_cast<const uint8_t *>(vrow);
#pragma unroll 4
    for (int pl = 0; pl < C; ++pl) {
      // Two code bytes: dims 4dq, 4dq+1 (low, high nibble of the first), 4dq+2, 4dq+3.
      const uint32_t c2 = *reinterpret_cast<const uint16_t *>(vb + ((size_t)pl * Hkv + gk) * (D / 2) + 2 * dq);
      const uint32_t lo = c2 & 0x0F0Fu, hi = (c2 >> 4) & 0x0F0Fu;
      const float u[4] = {(float)(lo & 0xFFu), (float)(hi & 0xFFu), (float)(lo >> 8), (float)(hi >> 8)};
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float w = wts[pl][gk * G + hh];
#pragma unroll
        for (int i = 0; i < 4; ++i) o[hh][i] = fmaf(w, u[i], o[hh][i]);
      }
    }
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const int h = gk * G + hh;
      const float ws8 = -8.0f * wsumh[h];
      float *dst = part_t + ((size_t)h * a.nchunks + chunk) * kPartStride;
      *reinterpret_cast<float4 *>(dst + 4 * dq) =
          float4{o[hh][0] + ws8, o[hh][1] + ws8, o[hh][2] + ws8, o[hh][3] + ws8};
    }
  }
}

// out[t][h][d] = sum_c exp(m_c - M) o_c[d] / sum_c exp(m_c - M) l_c over the
// chunks c, M = max_c m_c.  256 threads: thread (d = tid % 128, parity
// tid / 128) takes the chunks of its parity in index order, keeping a
// running maximum m and rescaling its two sums by exp(m_old - m_new)
// whenever a batch raises it (the same quotient; M never has to be known
// first, so every load of a batch goes out at once: one memory round trip
// up to 2B chunks), then the two parities are combined in a fixed order.
// Deterministic: the order of every operation is fixed.
template <int B>  // chunks per batch per thread
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a) {
  constexpr int D = kKvD;
  __shared__ float om[D], on[D], od[D];
  const int th = blockIdx.x, tid = threadIdx.x;  // th = t * Hq + h
  const int nc = a.nchunks;
  const float *p = a.part + (size_t)th * nc * kPartStride;
  const int d = tid & (D - 1), par = tid >> 7;
  float m = -INFINITY, num = 0.0f, den = 0.0f;
  for (int c0 = par; c0 < nc; c0 += 2 * B) {
    float v[B], l[B], mc[B];
#pragma unroll
    for (int i = 0; i < B; ++i) {
      const int c = c0 + 2 * i;
      const float *pc = p + (size_t)min(c, nc - 1) * kPartStride;
      v[i] = pc[d];
      l[i] = pc[D + 1];
      mc[i] = c < nc ? pc[D] : -INFINITY;  // past the end: weight 0
    }
    float mb = m;
#pragma unroll
    for (int i = 0; i < B; ++i) mb = fmaxf(mb, mc[i]);
    // Every chunk holds at least one position with a finite score, so mb is
    // finite from the first batch on; m is -inf only before it (sums 0).
    const float sc = m == -INFINITY ? 0.0f : __expf(m - mb);
    num *= sc;
    den *= sc;
#pragma unroll
    for (int i = 0; i < B; ++i) {
      const float w = __expf(mc[i] - mb);
      num = fmaf(w, v[i], num);
      den = fmaf(w, l[i], den);
    }
    m = mb;
  }
  if (par == 1) {
    om[d] = m;
    on[d] = num;
    od[d] = den;
  }
  __syncthreads();
  if (par == 0) {
    // Parity 1 is empty only with a single chunk (its m is then -inf).
    const float m1 = om[d], M = fmaxf(m, m1);
    const float f0 = __expf(m - M), f1 = m1 == -INFINITY ? 0.0f : __expf(m1 - M);
    a.out[(size_t)th * D + d] = (num * f0 + on[d] * f1) / (den * f0 + od[d] * f1);
  }
}

}  // namespace

bool kv_shape_supported(int Hkv, int D) { return D == kKvD && (Hkv == 1 || Hkv == 2 || Hkv == 4 || Hkv == 8); }

hipError_t launch_kv_quantize(const uint16_t *x, int T, int Hkv, const int *slots, int L, uint8_t *codes,
                              uint16_t *scale, hipStream_t s, const uint16_t *x2, uint8_t *codes2,
                              uint16_t *scale2) {
  KvQuantArgs a{};
  a.x[0] = x;
  a.codes[0] = codes;
  a.scale[0] = scale;
  a.x[1] = x2 ? x2 : x;
  a.codes[1] = x2 ? codes2 : codes;
  a.scale[1] = x2 ? scale2 : scale;
  a.rows1 = T * Hkv;
  a.rows = (x2 ? 2 : 1) * T * Hkv;
  a.Hkv = Hkv;
  a.L = L;
  a.slots = slots;
  KernelTimer timer("kv_quantize", s);
  kv_quantize_kernel<<<ceil_div(a.rows, 4 * kKvRowsPerWave), 256, 0, s>>>(a);
  return hipGetLastError();
}

size_t attn_workspace_bytes(int Tq, int Hq, int n_sel) {
  const long long nchunks = (n_sel + kAttnChunkMin - 1) / kAttnChunkMin;  // the larger count of the two chunk sizes
  return (size_t)Tq * Hq * nchunks * kPartStride * sizeof(float);
}

hipError_t launch_sparse_attention(const uint16_t *q, int Tq, int Hq, const uint8_t *kc, const uint16_t *ks,
                                   const uint8_t *vc, const uint16_t *vs, int L, int Hkv, const int *sel,
                                   int n_sel, float sm_scale, float *out, void *ws, hipStream_t s) {
  AttnArgs a{};
  a.q = q;
  a.kc = kc;
  a.vc = vc;
  a.ks = ks;
  a.vs = vs;
  a.sel = sel;
  a.Tq = Tq;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.L = L;
  a.n_sel = n_sel;
  const int C = attn_chunk(Tq, n_sel);
  a.nchunks = ceil_div(n_sel, C);
  a.sm_scale = sm_scale;
  a.part = static_cast<float *>(ws);
  a.out = out;
  const int G = Hq / Hkv;
  {
    KernelTimer timer("attn_partial", s);
    const dim3 grid((unsigned)(Tq * a.nchunks));
    auto go = [&](auto c) {
      constexpr int CC = decltype(c)::value;
      switch (G) {
        case 1: attn_partial_kernel<1, CC><<<grid, 256, 0, s>>>(a); break;
        case 2: attn_partial_kernel<2, CC><<<grid, 256, 0, s>>>(a); break;
        default: attn_partial_kernel<4, CC><<<grid, 256, 0, s>>>(a); break;
      }
    };
    if (C == kAttnChunkMax)
      go(std::integral_constant<int, kAttnChunkMax>{});
    else
      go(std::integral_constant<int, kAttnChunkMin>{});
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    KernelTimer timer("attn_merge", s);
    if (a.nchunks <= 32)
      attn_merge_kernel<16><<<dim3((unsigned)(Tq * Hq)), 256, 0, s>>>(a);
    else
      attn_merge_kernel<32><<<dim3((unsigned)(Tq * Hq)), 256, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace strata
