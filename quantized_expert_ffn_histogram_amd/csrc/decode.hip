// The whole routed FFN layer for a decode batch (T <= 16 tokens: one token
// plus drafts) in two kernels instead of route / group / gate-up / down /
// combine one after another.  At this size every kernel is a few
// microseconds of launch, first-load latency and drain around very little
// work, so the step time is set by the number of dependent kernels; each
// decode token is a fresh pass over its experts' weights ("两天移植，预填充
// 提速8倍：Strata引擎实测" (kongchang.com), section "Strata快在哪：不是魔法，
// 是物流"), bounded by memory bandwidth over the bytes read (lqnn.cn static
// review §4.1).
//
//   decode_route_gateup (grid: ceil(T/4) routing blocks + T*k*(I/16) others)
//     routing blocks: one wavefront per token selects its top-k and writes
//       topk_ids / topk_w exactly as the routing kernel does (same code);
//     the others: block (pair p = t*k + j, 16 h columns): each wavefront
//       re-selects the j-th expert of token t itself (same code, so the same
//       expert; no barrier before its weight loads), then streams that expert's gate and up rows for its columns and
//       writes h[p] = silu(gate . x_t) * (up . x_t) in fp16, pair order,
//       each 8 consecutive columns stored as the pairs (c, c+4) that the
//       dot products consume (h lives only between the two kernels);
//       The token's activations are loaded before the selection finishes.
//   decode_down_combine (grid: 1 grouping block + T * H/rows blocks)
//     grouping block: counts / offsets / perm / inv_perm from topk_ids with
//       the single-workgroup grouping of the grouping step (same code);
//     the others: block (token t, rows) stages h of the token's k pairs in
//       LDS with the sum of each 32-value chunk (once per block instead of
//       once per row), streams row n of each of its k experts' down weights and writes
//       out[t][n] = sum_j w[t][j] * (W_down[e_j][n] . h[t*k+j]), summed in j
//       order: deterministic, with no y round trip and no combine kernel.
//
// Dot products: fp16 pairs (1024 + u) against fp16 activations with
// v_dot2_f32_f16 and the exact offset correction per lane, as in the GEMV
// path (ffn_gemv.hip), except that the activations' odd pairs are held
// divided by 16 so that half of the nibbles need no shift (dot32_split).
// The other weight formats fold their zero points or fifth bits into the
// same dot products (dot32_fmt), with each lane's side data loaded beside its
// scale.
#include "gemv_dev.h"
#include "permute_dev.h"
#include "route_dev.h"

namespace strata {
namespace {

constexpr int kDecColsPerWave = 4;                 // h columns per wavefront
constexpr int kDecCols = 4 * kDecColsPerWave;      // h columns per workgroup
constexpr int kDecMaxChunks = kGemvMaxHidden / 2048;

struct DecodeArgs {
  const float *logits;  // fp32 [T][E]
  const uint16_t *x;    // bf16 [T][H]
  const uint8_t *gate, *up, *down;
  const uint16_t *gate_s, *up_s, *down_s;
  int T, H, I, g, k, E;
  int *ids;        // [T*k]
  float *w;        // [T*k]
  int *counts, *offsets, *perm, *inv_perm;
  uint16_t *h;     // fp16 [T*k][I], pair order
  float *out;      // fp32 [T][H]
  // Other weight formats: zero points or fifth-bit words of gate, up, down.
  const uint8_t *gate_x, *up_x, *down_x;
  int tiled;  // packed codes in 32-row x 128-K tiles (packed_offset), else row-major
};

template <int EPL, int NCH, int FMT>
__global__ __launch_bounds__(256) void decode_route_gateup_kernel(DecodeArgs a) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nroute = (a.T + 3) / 4;
  __shared__ TopkScratch sc[4];
  if ((int)blockIdx.x < nroute) {
    const int t = blockIdx.x * 4 + wave;
    if (t < a.T)
      wave_route_token<EPL>(a.logits + (size_t)t * a.E, a.E, a.k, a.ids + t * a.k, a.w + t * a.k, sc[wave]);
    return;
  }
  const int colsets = a.I / kDecCols;
  const int item = blockIdx.x - nroute, p = item / colsets, cs = item - p * colsets;
  const int t = p / a.k, j = p - t * a.k;

  // Lanes past H (H < 2048) load lane 0's data and get a zero scale.
  const bool active = 32 * lane < a.H;
  const int kl = active ? 32 * lane : 0;
  uint4 xv[NCH][4];
#pragma unroll
  for (int c = 0; c < NCH; ++c)
#pragma unroll
    for (int q = 0; q < 4; ++q) xv[c][q] = reinterpret_cast<const uint4 *>(a.x + (size_t)t * a.H + 2048 * c + kl)[q];

  // Every wavefront selects the expert itself (same code, same result), so
  // that no barrier stands between the selection and its weight loads.
  int my_id;
  float my_val;
  wave_topk<EPL>(a.logits + (size_t)t * a.E, a.E, j + 1, my_id, my_val, sc[wave]);
  const int e = __builtin_amdgcn_readlane(my_id, j);

  const int kb = a.H / 2, ng = a.H / a.g;
  const int n0 = cs * kDecCols + wave * kDecColsPerWave;
  uint4 wg[kDecColsPerWave][NCH], wu[kDecColsPerWave][NCH];
  uint32_t sgb[kDecColsPerWave][NCH], sub_[kDecColsPerWave][NCH];
  uint32_t xg[kDecColsPerWave][NCH], xu[kDecColsPerWave][NCH];  // side data of the other formats
#pragma unroll
  for (int cc = 0; cc < kDecColsPerWave; ++cc)
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const size_t row = (size_t)e * a.I + n0 + cc;
      const int kk = 2048 * c + kl;
      const size_t wo = packed_offset(row, (uint32_t)(kk / 2), (uint32_t)kb, a.tiled != 0);
      wg[cc][c] = *reinterpret_cast<const uint4 *>(a.gate + wo);
      wu[cc][c] = *reinterpret_cast<const uint4 *>(a.up + wo);
      sgb[cc][c] = a.gate_s[row * ng + kk / a.g];
      sub_[cc][c] = a.up_s[row * ng + kk / a.g];
      xg[cc][c] = gemv_aux<FMT>(a.gate_x, row, a.H, a.g, kk);
      xu[cc][c] = gemv_aux<FMT>(a.up_x, row, a.H, a.g, kk);
    }
  const float on = active ? 1.0f : 0.0f;
  float gs[kDecColsPerWave], us[kDecColsPerWave];
#pragma unroll
  for (int cc = 0; cc < kDecColsPerWave; ++cc) gs[cc] = us[cc] = 0.0f;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    half2_t xp[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) bf16x8_pairs(xv[c][q], &xp[4 * q]);
    // Odd pairs divided by 16 (dot32_split), once for the wavefront's 8 rows.
    const half2_t sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
    float se = 0.0f, so = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      xp[4 * q + 1] *= sixteenth;
      xp[4 * q + 3] *= sixteenth;
      se += pair_sum(xp[4 * q]) + pair_sum(xp[4 * q + 2]);
      so += pair_sum(xp[4 * q + 1]) + pair_sum(xp[4 * q + 3]);
    }
    const float corr = 1032.0f * se + 1152.0f * so;
#pragma unroll
    for (int cc = 0; cc < kDecColsPerWave; ++cc) {
      const float sg = on * half_bits_to_float((uint16_t)sgb[cc][c]);
      const float su = on * half_bits_to_float((uint16_t)sub_[cc][c]);
      if constexpr (FMT == 0) {
        gs[cc] += dot32_split<false>(wg[cc][c], xp, corr, sg);
        us[cc] += dot32_split<false>(wu[cc][c], xp, corr, su);
      } else {
        gs[cc] += dot32_fmt<false, FMT>(wg[cc][c], xp, se, so, sg, xg[cc][c]);
        us[cc] += dot32_fmt<false, FMT>(wu[cc][c], xp, se, so, su, xu[cc][c]);
      }
    }
  }
#pragma unroll
  for (int cc = 0; cc < kDecColsPerWave; ++cc) {
    const float gv = dpp_group_sum<kWave>(gs[cc]);
    const float uv = dpp_group_sum<kWave>(us[cc]);
    if (lane == 0) {
      const float hv = gv / (1.0f + __expf(-gv)) * uv;
      // Pair order (c, c+4); the odd pairs (c % 4 = 1, 3) divided by 16 for dot32_split.
      const int c = n0 + cc, slot = (c & ~7) | (2 * (c & 3) + ((c >> 2) & 1));
      reinterpret_cast<_Float16 *>(a.h)[(size_t)p * a.I + slot] = (_Float16)((c & 1) ? hv * 0.0625f : hv);
    }
  }
}

template <int LPR, int KMAX, int FMT>  // lanes per down row = I / 32; KMAX >= k
__global__ __launch_bounds__(256) void decode_down_combine_kernel(DecodeArgs a) {
  constexpr int RPW = kWave / LPR;  // rows per wavefront
  constexpr int kRowsWG = 4 * RPW;  // output rows per workgroup
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (blockIdx.x == 0) {
    group_small(a.ids, a.T * a.k, a.E, a.counts, a.offsets, a.perm, a.inv_perm);
    return;
  }
  const int sub = lane % LPR, rsel = lane / LPR;
  const int rowsets = (a.H + kRowsWG - 1) / kRowsWG;
  const int item = blockIdx.x - 1, t = item / rowsets, rs = item - t * rowsets;
  const int n = rs * kRowsWG + wave * RPW + rsel;  // this lane's output row
  const int nc = n < a.H ? n : 0;                  // rows past H load row 0 and are not stored

  // Lane j (< k) holds pair j's expert and routing weight.
  const int pj = t * a.k + (lane < a.k ? lane : 0);
  const int eid = a.ids[pj];
  const float wj = lane < a.k ? a.w[pj] : 0.0f;

  // h of the token's k pairs (fp16, k * I <= kDecodeMaxKI values) does not
  // depend on the routing: it goes straight to LDS with direct-to-LDS loads
  // through a buffer resource (range-checked: slots past k * I read zeros),
  // issued right after the routing loads (so waiting for those does not wait
  // for h) and in flight with the weight loads.
  constexpr int kHLoads = kDecodeMaxKI / 8 / 256;  // 16-byte loads per thread
  __shared__ uint4 hs[kDecodeMaxKI / 8];
  {
    const __amdgpu_buffer_rsrc_t rh = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(a.h + (size_t)t * a.k * a.I), 0, a.k * a.I * 2, 0x00020000);
#pragma unroll
    for (int i = 0; i < kHLoads; ++i) {
      const int slot = 256 * i + 64 * wave;  // first uint4 slot of this wavefront's load
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rh, (__attribute__((address_space(3))) void *)&hs[slot], 16,
                                               (uint32_t)(slot + lane) * 16u, 0, 0, 0);
    }
  }
  asm volatile("" ::: "memory");  // the weight loads below are issued after the h loads

  // Row n of each pair's expert: this lane's 32 K values (16 bytes) and their scale.
  const int kb = a.I / 2, ng = a.I / a.g;
  uint4 wq[KMAX];
  uint32_t sdb[KMAX], xd[KMAX];
#pragma unroll
  for (int jj = 0; jj < KMAX; ++jj) {
    const int e = __builtin_amdgcn_readlane(eid, jj < a.k ? jj : a.k - 1);  // past k: repeat the last row
    const size_t row = (size_t)e * a.H + nc;
    wq[jj] = *reinterpret_cast<const uint4 *>(a.down + packed_offset(row, 16u * sub, (uint32_t)kb, a.tiled != 0));
    sdb[jj] = a.down_s[row * ng + (32 * sub) / a.g];
    xd[jj] = gemv_aux<FMT>(a.down_x, row, a.I, a.g, 32 * sub);
  }
  // This wavefront's h loads have landed once no more than the loads issued
  // after them are outstanding: per expert slot a weight row and a scale,
  // and for the other formats their side data.  The weight stream goes on
  // during the chunk sums below, and the dot products wait per expert.
  constexpr int kYounger = (FMT == 0 ? 2 : 3) * KMAX;
  static_assert(kYounger < 64, "vmcnt range");
  asm volatile("" ::: "memory");  // every load above is issued before the wait
  __builtin_amdgcn_s_waitcnt((kYounger & 0xF) | ((kYounger >> 4) << 14) | 0x0F70);
  asm volatile("" ::: "memory");
  __syncthreads();  // ... and everyone's
  // Sum of each 32-value chunk of h (the offset correction of the dot
  // products), once per chunk: thread tid sums chunks tid, tid + 256, ...
  __shared__ float hsums[kDecodeMaxKI / 32];
  __shared__ float hse[FMT == 0 ? 1 : kDecodeMaxKI / 32], hso[FMT == 0 ? 1 : kDecodeMaxKI / 32];
  for (int c = tid; c < a.k * a.I / 32; c += 256) {
    const uint4 *hc = hs + 4 * c;
    float se = 0.0f, so = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 u = hc[q];
      se += pair_sum(__builtin_bit_cast(half2_t, u.x)) + pair_sum(__builtin_bit_cast(half2_t, u.z));
      so += pair_sum(__builtin_bit_cast(half2_t, u.y)) + pair_sum(__builtin_bit_cast(half2_t, u.w));
    }
    hsums[c] = 1032.0f * se + 1152.0f * so;  // the offset term of dot32_split
    if constexpr (FMT != 0) {  // the other formats' offset terms need both sums
      hse[c] = se;
      hso[c] = so;
    }
  }
  __syncthreads();

  float acc = 0.0f;
#pragma unroll
  for (int jj = 0; jj < KMAX; ++jj) {
    if (jj < a.k) {
      // h is stored in pair order: each 32-bit word is one fp16 pair.
      const uint4 *hrow = hs + (jj * a.I + 32 * sub) / 8;
      half2_t hp[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 u = hrow[q];
        hp[4 * q] = __builtin_bit_cast(half2_t, u.x);
        hp[4 * q + 1] = __builtin_bit_cast(half2_t, u.y);
        hp[4 * q + 2] = __builtin_bit_cast(half2_t, u.z);
        hp[4 * q + 3] = __builtin_bit_cast(half2_t, u.w);
      }
      const int hc = (jj * a.I) / 32 + sub;
      const float wsel = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wj), jj));
      const float sd = half_bits_to_float((uint16_t)sdb[jj]);
      if constexpr (FMT == 0)
        acc += wsel * dot32_split<true>(wq[jj], hp, hsums[hc], sd);
      else
        acc += wsel * dot32_fmt<true, FMT>(wq[jj], hp, hse[hc], hso[hc], sd, xd[jj]);
    }
  }
  const float y = dpp_group_sum<LPR>(acc);
  if (sub == 0 && n < a.H) a.out[(size_t)t * a.H + n] = y;
}

// Row loads past k repeat the last expert's row: instances for k up to 4, 6,
// 8, 10, 12 and 16 keep them to at most two per lane for k <= 12 and none at
// k = 10 (0.2 us less per decode step than 12 rows).
template <int LPR, int FMT>
void launch_down_combine(const DecodeArgs &a, int grid, hipStream_t s) {
  if (a.k <= 4)
    decode_down_combine_kernel<LPR, 4, FMT><<<grid, 256, 0, s>>>(a);
  else if (a.k <= 6)
    decode_down_combine_kernel<LPR, 6, FMT><<<grid, 256, 0, s>>>(a);
  else if (a.k <= 8)
    decode_down_combine_kernel<LPR, 8, FMT><<<grid, 256, 0, s>>>(a);
  else if (a.k <= 10)
    decode_down_combine_kernel<LPR, 10, FMT><<<grid, 256, 0, s>>>(a);
  else if (a.k <= 12)
    decode_down_combine_kernel<LPR, 12, FMT><<<grid, 256, 0, s>>>(a);
  else
    decode_down_combine_kernel<LPR, 16, FMT><<<grid, 256, 0, s>>>(a);
}

template <int NCH, int FMT>
void launch_route_gateup(const DecodeArgs &a, int grid, hipStream_t s) {
  if (a.E <= 64)
    decode_route_gateup_kernel<1, NCH, FMT><<<grid, 256, 0, s>>>(a);
  else if (a.E <= 128)
    decode_route_gateup_kernel<2, NCH, FMT><<<grid, 256, 0, s>>>(a);
  else if (a.E <= 256)
    decode_route_gateup_kernel<4, NCH, FMT><<<grid, 256, 0, s>>>(a);
  else if (a.E <= 512)
    decode_route_gateup_kernel<8, NCH, FMT><<<grid, 256, 0, s>>>(a);
  else
    decode_route_gateup_kernel<16, NCH, FMT><<<grid, 256, 0, s>>>(a);
}

// The two kernels of one weight format.
template <int FMT>
void launch_decode_kernels(const DecodeArgs &a, int T, int k, const FfnWeights &w, hipStream_t s, hipError_t &err) {
  {
    KernelTimer timer("decode_route_gateup", s);
    const int grid = (T + 3) / 4 + T * k * (w.I / kDecCols);
    if (w.H <= 2048)
      launch_route_gateup<1, FMT>(a, grid, s);
    else
      launch_route_gateup<kDecMaxChunks, FMT>(a, grid, s);
  }
  if ((err = hipGetLastError()) != hipSuccess) return;
  {
    KernelTimer timer("decode_down_combine", s);
    const int lpr = w.I / 32;
    const int rows_wg = 4 * (kWave / lpr);
    const int grid = 1 + T * ((w.H + rows_wg - 1) / rows_wg);
    switch (lpr) {
      case 4: launch_down_combine<4, FMT>(a, grid, s); break;
      case 8: launch_down_combine<8, FMT>(a, grid, s); break;
      case 16: launch_down_combine<16, FMT>(a, grid, s); break;
      case 32: launch_down_combine<32, FMT>(a, grid, s); break;
      default: launch_down_combine<64, FMT>(a, grid, s); break;
    }
  }
  err = hipGetLastError();
}

}  // namespace

bool decode_layer_supported(int T, int E, int k, int H, int I) {
  return T >= 1 && T <= kGemvMaxTokens && k <= kDecodeMaxK && E <= kMaxExperts && (long long)k * I <= kDecodeMaxKI &&
         gemv_supported(T, H, I);
}

hipError_t launch_decode_layer(const float *logits, const uint16_t *x, int T, int k, const FfnWeights &w,
                               int *ids, float *topk_w, int *counts, int *offsets, int *perm, int *inv_perm,
                               float *out, const FfnWorkspace &ws, hipStream_t s) {
  DecodeArgs a{};
  a.logits = logits;
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
  a.E = w.E;
  a.ids = ids;
  a.w = topk_w;
  a.counts = counts;
  a.offsets = offsets;
  a.perm = perm;
  a.inv_perm = inv_perm;
  a.h = ws.h;
  a.out = out;
  a.gate_x = w.gate_x;
  a.up_x = w.up_x;
  a.down_x = w.down_x;
  a.tiled = w.tiled;
  hipError_t err = hipSuccess;
  if (w.fmt == 1)
    launch_decode_kernels<1>(a, T, k, w, s, err);
  else if (w.fmt == 2)
    launch_decode_kernels<2>(a, T, k, w, s, err);
  else
    launch_decode_kernels<0>(a, T, k, w, s, err);
  return err;
}

}  // namespace strata
