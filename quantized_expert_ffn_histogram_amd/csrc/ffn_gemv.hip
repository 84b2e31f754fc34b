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
// experts selected this step are touched.
//
// Work list: entry i is the i-th expert (in index order) with a non-zero
// count; every workgroup finds its expert from the offsets itself (a block
// scan of the non-empty flags), so no planning kernel runs first.  An expert
// holds at most T <= 16 pairs here (a token picks an expert at most once);
// its weights are loaded into registers once and applied to its rows one
// after another.  All weight loads of a wavefront are issued before any arithmetic,
// so each lane has 8 (gate/up) or 8 (down) 16-byte loads in flight.
//
// Dot products: a dword of 8 nibbles gives four fp16 pairs (1024 + u_m,
// 1024 + u_{m+4}) with one and-or each (and one shift per dword: the pairs
// from bits 4..7 of each byte are used in place as 1024 + 16u against
// activations divided by 16, dot32_split); v_dot2_f32_f16 accumulates in
// fp32, and per lane (32 K values, inside one group since g >= 32) the exact
// identity  sum x*q*s = s * (acc - offset term)  removes the offset.
// Activations are converted to fp16 pairs in the same slot order; h between
// the two kernels is stored in that order already.
//
//   gemv_gateup: workgroup = (entry, 16 h columns); wavefront = 4 columns,
//                gate and up rows; lane 0 writes h = silu(g)*u (fp16).
//   gemv_down:   workgroup = (entry, 1024/(I/32) output rows); each output
//                row is reduced over I/32 lanes.  Fused combine: y goes to
//                fp16 rows in pair order and the combine kernel of the
//                matrix-core path sums each token's k rows in j order
//                (deterministic, no atomics).
#include <type_traits>

#include "gemv_dev.h"

namespace strata {
namespace {

// Tile sizes measured best on the decode shape (T=4, H=2048, I=512, E=512,
// k=10) among 2/4/8 columns per wavefront and 1/2/4/8/16 down loads per lane.
constexpr int kColsPerWave = 4;                // h columns per wavefront
constexpr int kGateUpCols = 4 * kColsPerWave;  // h columns per workgroup
constexpr int kDownIter = 4;   // 16-byte weight loads per lane in gemv_down
constexpr int kMaxChunks = kGemvMaxHidden / 2048;

struct GemvArgs {
  const uint16_t *x;      // bf16 [T][H]
  const uint8_t *gate, *up, *down;
  const uint16_t *gate_s, *up_s, *down_s;
  int T, H, I, g, k, E;
  const int *offsets;     // [E+1]
  const int *perm;
  const float *topk_w;
  uint16_t *h;            // fp16 [pairs][I], grouped order
  float *out;             // not fused: y [pairs][H] in grouped order
  uint16_t *y16;          // fused: fp16 y [pairs][H] in pair order, summed by the combine kernel
  int fused;
  // Other weight formats: zero points (two per byte, [E][N][K/g/2]) or
  // fifth-bit words ([E][N][K/32]) of gate, up and down.
  const uint8_t *gate_x, *up_x, *down_x;
  int tiled;  // packed codes in 32-row x 128-K tiles (packed_offset), else row-major
};


struct Entry {
  int e, row0, rows, nnz;  // e < 0: no such entry
};

// The `entry`-th expert with a non-zero count (experts in index order) and the
// number of such experts.  Block-wide (256 threads, E <= 1024), uniform result.
__device__ Entry find_entry(const int *__restrict__ offsets, int E, int entry) {
  __shared__ int wave_tot[4];
  __shared__ Entry found;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int lo[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) lo[i] = offsets[min(4 * tid + i, E)];  // unconditional loads, clamped
  int cnt = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) cnt += (4 * tid + i < E && lo[i + 1] > lo[i]) ? 1 : 0;
  int incl = cnt;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int v = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += v;
  }
  if (lane == kWave - 1) wave_tot[wave] = incl;
  if (tid == 0) found = Entry{-1, 0, 0, 0};
  __syncthreads();
  int base = 0, nnz = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    base += w < wave ? wave_tot[w] : 0;
    nnz += wave_tot[w];
  }
  int r = entry - (base + incl - cnt);
  if (r >= 0 && r < cnt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool nz = 4 * tid + i < E && lo[i + 1] > lo[i];
      if (nz && r == 0) found = Entry{4 * tid + i, lo[i], lo[i + 1] - lo[i], 0};
      r -= nz ? 1 : 0;
    }
  }
  __syncthreads();
  Entry out = found;
  out.nnz = nnz;
  return out;
}

// A lane covers K values [32*lane + 2048*c, +32) for c < NCH = ceil(H/2048)
// (only the first H/32 lanes when H < 2048).
template <int NCH, int FMT>
__global__ __launch_bounds__(256, NCH == 1 ? 4 : 2) void gemv_gateup_kernel(GemvArgs a) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int colsets = a.I / kGateUpCols;
  const int entry = blockIdx.x / colsets, cs = blockIdx.x - entry * colsets;
  const Entry en = find_entry(a.offsets, a.E, entry);
  if (en.e < 0) return;

  // Lanes past H (H < 2048) load lane 0's data and get a zero scale, so every
  // load is unconditional and all of them are in flight together.
  const bool active = 32 * lane < a.H;
  const int kl = active ? 32 * lane : 0;
  const int kb = a.H / 2, ng = a.H / a.g;
  const int n0 = cs * kGateUpCols + wave * kColsPerWave;

  // The first row's pair index is loaded before the weights: vector loads
  // complete in order, so the x loads that depend on it wait only for it.
  int p_first = a.perm[en.row0];
  // This wavefront's gate and up rows (4 columns) and their scales (fp16 bits).
  uint4 wg[kColsPerWave][NCH], wu[kColsPerWave][NCH];
  uint32_t sgb[kColsPerWave][NCH], sub_[kColsPerWave][NCH];
  uint32_t xg[kColsPerWave][NCH], xu[kColsPerWave][NCH];  // side data of the other formats
#pragma unroll
  for (int cc = 0; cc < kColsPerWave; ++cc)
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const size_t row = (size_t)en.e * a.I + n0 + cc;
      const int kk = 2048 * c + kl;
      const size_t wo = packed_offset(row, (uint32_t)(kk / 2), (uint32_t)kb, a.tiled != 0);
      wg[cc][c] = *reinterpret_cast<const uint4 *>(a.gate + wo);
      wu[cc][c] = *reinterpret_cast<const uint4 *>(a.up + wo);
      sgb[cc][c] = a.gate_s[row * ng + kk / a.g];
      sub_[cc][c] = a.up_s[row * ng + kk / a.g];
      xg[cc][c] = gemv_aux<FMT>(a.gate_x, row, a.H, a.g, kk);
      xu[cc][c] = gemv_aux<FMT>(a.up_x, row, a.H, a.g, kk);
    }
  asm volatile("" : "+v"(p_first) : : "memory");  // all of the above are issued before p_first is used
  const float on = active ? 1.0f : 0.0f;

  auto one_row = [&](int t, int r) {
    uint4 xv[NCH][4];
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        xv[c][q] = reinterpret_cast<const uint4 *>(a.x + (size_t)t * a.H + 2048 * c + kl)[q];
    // One wait for this row's x loads (issued together); the weights and
    // scales are pinned here too (see opaque()).
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
      for (int q = 0; q < 4; ++q) opaque(xv[c][q]);
#pragma unroll
    for (int cc = 0; cc < kColsPerWave; ++cc)
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        opaque(wg[cc][c]);
        opaque(wu[cc][c]);
        asm volatile("" : "+v"(sgb[cc][c]), "+v"(sub_[cc][c]));
        if constexpr (FMT != 0) asm volatile("" : "+v"(xg[cc][c]), "+v"(xu[cc][c]));
      }
    float gs[kColsPerWave], us[kColsPerWave];
#pragma unroll
    for (int cc = 0; cc < kColsPerWave; ++cc) gs[cc] = us[cc] = 0.0f;
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
      for (int cc = 0; cc < kColsPerWave; ++cc) {
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
    for (int cc = 0; cc < kColsPerWave; ++cc) {
      const float gv = dpp_group_sum<kWave>(gs[cc]);
      const float uv = dpp_group_sum<kWave>(us[cc]);
      if (lane == 0) {
        const float hv = gv / (1.0f + __expf(-gv)) * uv;
        // Pair order (c, c+4) inside each 8 columns, odd pairs divided by 16 (dot32_split).
        const int col = n0 + cc, slot = (col & ~7) | (2 * (col & 3) + ((col >> 2) & 1));
        reinterpret_cast<_Float16 *>(a.h)[(size_t)(en.row0 + r) * a.I + slot] =
            (_Float16)((col & 1) ? hv * 0.0625f : hv);
      }
    }
  };
  one_row(p_first / a.k, 0);
  for (int r = 1; r < en.rows; ++r) one_row(a.perm[en.row0 + r] / a.k, r);
}

template <int LPR, int FMT>  // lanes per down row = I / 32
__global__ __launch_bounds__(256, 4) void gemv_down_kernel(GemvArgs a) {
  constexpr int RPI = kWave / LPR;              // rows per wavefront instruction
  constexpr int kRowsWG = 4 * kDownIter * RPI;  // output rows per workgroup
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = lane % LPR, rsel = lane / LPR;
  const int nslices = (a.H + kRowsWG - 1) / kRowsWG;
  const int entry = blockIdx.x / nslices, slice = blockIdx.x - entry * nslices;
  const Entry en = find_entry(a.offsets, a.E, entry);
  if (en.e < 0) return;

  const int kb = a.I / 2, ng = a.I / a.g;
  const int nbase = slice * kRowsWG + wave * kDownIter * RPI + rsel;  // row of iteration it: nbase + it*RPI

  // Row r's h fragment (fp16, 32 values per lane) and output row; the first
  // row's are issued before the weights.
  auto load_row = [&](int r, uint4 (&hv)[4], int &dst) {
    const int gi = en.row0 + r;
    dst = a.fused ? a.perm[gi] : gi;
    const uint4 *src = reinterpret_cast<const uint4 *>(a.h + (size_t)gi * a.I + 32 * sub);
#pragma unroll
    for (int q = 0; q < 4; ++q) hv[q] = src[q];
  };
  uint4 hv[4];
  int dst;
  load_row(0, hv, dst);

  // Rows past H (only when H is below the workgroup's row count) load row 0 and are not stored.
  uint4 wq[kDownIter];
  uint32_t sdb[kDownIter], xd[kDownIter];
#pragma unroll
  for (int it = 0; it < kDownIter; ++it) {
    const int n = nbase + it * RPI;
    const size_t row = (size_t)en.e * a.H + (n < a.H ? n : 0);
    wq[it] = *reinterpret_cast<const uint4 *>(a.down + packed_offset(row, 16u * sub, (uint32_t)kb, a.tiled != 0));
    sdb[it] = a.down_s[row * ng + (32 * sub) / a.g];
    xd[it] = gemv_aux<FMT>(a.down_x, row, a.I, a.g, 32 * sub);
  }

  for (int r = 0; r < en.rows; ++r) {
    if (r > 0) load_row(r, hv, dst);
#pragma unroll
    for (int q = 0; q < 4; ++q) opaque(hv[q]);
#pragma unroll
    for (int it = 0; it < kDownIter; ++it) {
      opaque(wq[it]);
      asm volatile("" : "+v"(sdb[it]));
    }
    // h is stored in pair order with the odd pairs divided by 16: each
    // 32-bit word is one pair for dot32_split.
    half2_t hp[16];
    float se = 0.0f, so = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      hp[4 * q] = __builtin_bit_cast(half2_t, hv[q].x);
      hp[4 * q + 1] = __builtin_bit_cast(half2_t, hv[q].y);
      hp[4 * q + 2] = __builtin_bit_cast(half2_t, hv[q].z);
      hp[4 * q + 3] = __builtin_bit_cast(half2_t, hv[q].w);
      se += pair_sum(hp[4 * q]) + pair_sum(hp[4 * q + 2]);
      so += pair_sum(hp[4 * q + 1]) + pair_sum(hp[4 * q + 3]);
    }
    const float corr = 1032.0f * se + 1152.0f * so;
#pragma unroll
    for (int it = 0; it < kDownIter; ++it) {
      const float sd = half_bits_to_float((uint16_t)sdb[it]);
      const float yv = dpp_group_sum<LPR>(FMT == 0 ? dot32_split<true>(wq[it], hp, corr, sd)
                                                   : dot32_fmt<true, FMT>(wq[it], hp, se, so, sd, xd[it]));
      const int n = nbase + it * RPI;
      if (sub == 0 && n < a.H) {
        if (a.fused)
          reinterpret_cast<_Float16 *>(a.y16)[(size_t)dst * a.H + n] = (_Float16)yv;
        else
          a.out[(size_t)dst * a.H + n] = yv;
      }
    }
  }
}

}  // namespace

bool gemv_supported(int T, int H, int I) {
  const bool pow2 = I >= 128 && I <= 2048 && (I & (I - 1)) == 0;
  return T <= kGemvMaxTokens && H <= kGemvMaxHidden && (H & (H - 1)) == 0 && pow2;
}

hipError_t launch_ffn_gemv(const uint16_t *x, int T, int k, const FfnWeights &w, const int *offsets,
                           const int *perm, const float *topk_w, float *y_or_out,
                           const FfnWorkspace &ws, hipStream_t s) {
  const int entries = (int)std::min<long long>((long long)T * k, w.E);
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
  a.E = w.E;
  a.offsets = offsets;
  a.perm = perm;
  a.topk_w = topk_w;
  a.h = ws.h;
  a.out = y_or_out;
  a.y16 = ws.y16;
  a.fused = topk_w != nullptr;
  a.gate_x = w.gate_x;
  a.up_x = w.up_x;
  a.down_x = w.down_x;
  a.tiled = w.tiled;
  {
    KernelTimer timer("gemv_gateup", s);
    const int grid = entries * (w.I / kGateUpCols);
    auto go = [&](auto fc) {
      constexpr int F = decltype(fc)::value;
      if (w.H <= 2048)
        gemv_gateup_kernel<1, F><<<grid, 256, 0, s>>>(a);
      else
        gemv_gateup_kernel<kMaxChunks, F><<<grid, 256, 0, s>>>(a);
    };
    if (w.fmt == 1)
      go(std::integral_constant<int, 1>{});
    else if (w.fmt == 2)
      go(std::integral_constant<int, 2>{});
    else
      go(std::integral_constant<int, 0>{});
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int lpr = w.I / 32;
  const int rows_wg = 4 * kDownIter * (kWave / lpr);
  const int grid = entries * ((w.H + rows_wg - 1) / rows_wg);
  {
    KernelTimer timer("gemv_down", s);
    auto go = [&](auto fc) {
      constexpr int F = decltype(fc)::value;
      switch (lpr) {
        case 4: gemv_down_kernel<4, F><<<grid, 256, 0, s>>>(a); break;
        case 8: gemv_down_kernel<8, F><<<grid, 256, 0, s>>>(a); break;
        case 16: gemv_down_kernel<16, F><<<grid, 256, 0, s>>>(a); break;
        case 32: gemv_down_kernel<32, F><<<grid, 256, 0, s>>>(a); break;
        default: gemv_down_kernel<64, F><<<grid, 256, 0, s>>>(a); break;
      }
    };
    if (w.fmt == 1)
      go(std::integral_constant<int, 1>{});
    else if (w.fmt == 2)
      go(std::integral_constant<int, 2>{});
    else
      go(std::integral_constant<int, 0>{});
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (a.fused) return launch_combine_pairs(ws.y16, topk_w, T, k, w.H, y_or_out, s);
  return hipSuccess;
}

}  // namespace strata
