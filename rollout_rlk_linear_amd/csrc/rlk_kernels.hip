// rlk_kernels.hip — gfx950 kernels of the fused, batch-invariant linear log-prob.
//
// Forward (per call):
//   fwd_tile     one workgroup per (T-tile, vocabulary group of 256 columns):
//                bf16 MFMA logits for the tile, kept in registers; per row and
//                32-column chunk the statistics (m, R, B) by a fixed 16-lane
//                DPP tree; the 8 chunks of the group folded left to right;
//                one (m, R, B, zy) record per (row, group) written to the
//                workspace. No T x V logits ever reach memory.
//   fwd_combine  one wave per row: the row's group records folded in a fixed
//                lane-strided order plus a fixed 64-lane tree; writes logp,
//                entropy and the row's statistics record.
// Backward (per vocabulary chunk, chunks made of whole dH splits):
//   bwd_rowprep    per row: log1p(R), -B/(1+R), upstream gradients, local target.
//   bwd_recompute  logits of the chunk again (same MFMA chain as the forward,
//                  so the same bits), the logit gradient G in fp32, RNE to
//                  bf16, staged through LDS and stored [T][chunk] coalesced.
//   bwd_dw         dW[v, :] = sum_t G[t, v] h[t, :]  (both operands K-strided,
//                  transposed in registers), fp32, one owner per element.
//   bwd_dh         dH partial of split s = sum_{v in s} G[t, v] W[v, :], one
//                  MFMA chain over the split in ascending v; splits are set by
//                  V alone.
//   bwd_dh_reduce  dH = sum_s partial_s in the order s = 0, 1, ...; bf16 RNE or fp32.
// Nothing uses atomics. All per-row arithmetic is independent of the tile
// shape and the grid, so every row's outputs are identical for any T.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rlk_device.cuh"
#include "rlk_internal.h"

namespace rlk {

// Decode a linear block id into (group, T-tile) so that all T-tiles of one
// group run on the same XCD (workgroups are dealt to the 8 XCDs round-robin)
// and share the group's W tile in that XCD's L2.
__device__ __forceinline__ void xcd_decode(int b, int n_ttiles, int& g, int& tt) {
  const int xcd = b & 7;
  const int seq = b >> 3;
  g = xcd + 8 * (seq / n_ttiles);
  tt = seq % n_ttiles;
}

// ======================================================= forward tile ====

template <int BM, int WM, int WN>
__global__ __launch_bounds__(kThreads) void fwd_tile_kernel(
    const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ weight,
    const int32_t* __restrict__ targets, int T, int H, int V, int64_t vocab_start, int G,
    int n_ttiles, float4* __restrict__ part) {
  using Gm = AsyncGemm<BM, GROUP, WM, WN>;
  static_assert(BM * CHUNKS_PER_GROUP * 3 * 4 <= Gm::LDS_BYTES, "chunk stats fit in the stages");
  __shared__ __attribute__((aligned(16))) unsigned char lds[Gm::LDS_BYTES];
  __shared__ int ycol[BM];
  __shared__ float zys[BM];

  int g, tt;
  xcd_decode(blockIdx.x, n_ttiles, g, tt);
  if (g >= G) return;
  const int row0 = tt * BM;
  const int col0 = g * GROUP;
  const int tid = threadIdx.x;
  if (tid < BM) {
    const int t = row0 + tid;
    int yc = -1;
    if (t < T) {
      const int64_t y = (int64_t)targets[t] - vocab_start - col0;
      if (y >= 0 && y < GROUP && y < (int64_t)(V - col0)) yc = (int)y;
    }
    ycol[tid] = yc;
    zys[tid] = neg_inf();
  }

  Gm gm;
  gm.zero();
  gm.run(lds, hidden + (int64_t)row0 * H, H, T - row0, weight + (int64_t)col0 * H, H, V - col0, 0,
         H);
  // run() ends on a barrier: the LDS stages are free and ycol/zys are visible.

  float* cst = reinterpret_cast<float*>(lds);  // [BM][8 chunks][3]
  const int lane = tid & 63;
  const int wave = wave_id();
  const int wm = wave % WM, wn = wave / WM;
  const int vlim = V - col0;
#pragma unroll
  for (int i = 0; i < Gm::MI; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int rl = wm * Gm::WTM + 16 * i + 4 * (lane >> 4) + r;
      const int yc = ycol[rl];
#pragma unroll
      for (int q = 0; q < Gm::NJ / 2; ++q) {
        const int c0 = wn * Gm::WTN + CHUNK * q + (lane & 15);
        const int c1 = c0 + 16;
        const bool va = c0 < vlim, vb = c1 < vlim;
        const float za = va ? gm.acc[i][2 * q][r] : neg_inf();
        const float zb = vb ? gm.acc[i][2 * q + 1][r] : neg_inf();
        if (c0 == yc) zys[rl] = za;
        if (c1 == yc) zys[rl] = zb;
        // chunk = columns c0 and c1 of the 16 lanes of this row group
        const float m = row16_max(fmaxf(za, zb));
        const bool ta = va && za == m, tb = vb && zb == m;
        const int nties = row16_sum_i((int)ta + (int)tb);
        const float da = va ? za - m : 0.f;
        const float db = vb ? zb - m : 0.f;
        const float ea = (ta || !va) ? 0.f : exp_fast(da);
        const float eb = (tb || !vb) ? 0.f : exp_fast(db);
        const float R = row16_sum(ea + eb) + (float)(nties - 1);
        const float B = row16_sum(ea * da + eb * db);
        if ((lane & 15) == 0) {
          float* p = cst + (rl * CHUNKS_PER_GROUP + wn * (Gm::WTN / CHUNK) + q) * 3;
          p[0] = m;
          p[1] = R;
          p[2] = B;
        }
      }
    }
  }
  __syncthreads();
  if (tid < BM && row0 + tid < T) {
    const int nvc = min(CHUNKS_PER_GROUP, (vlim + CHUNK - 1) / CHUNK);
    const float* p = cst + tid * CHUNKS_PER_GROUP * 3;
    Part acc{p[0], p[1], p[2], neg_inf()};
    for (int c = 1; c < nvc; ++c) acc = part_merge(acc, Part{p[3 * c], p[3 * c + 1], p[3 * c + 2], neg_inf()});
    acc.zy = zys[tid];
    part[(int64_t)(row0 + tid) * G + g] = make_float4(acc.m, acc.R, acc.B, acc.zy);
  }
}

// ==================================================== forward combine ====

__device__ __forceinline__ Part shfl_xor_part(const Part& p, int s) {
  return Part{__shfl_xor(p.m, s), __shfl_xor(p.R, s), __shfl_xor(p.B, s), __shfl_xor(p.zy, s)};
}

__global__ __launch_bounds__(kThreads) void fwd_combine_kernel(
    const float4* __restrict__ part, const int32_t* __restrict__ targets, int T, int G,
    int64_t vocab_total, int full, float* __restrict__ logp, float* __restrict__ entropy,
    float4* __restrict__ stats) {
  const int row = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= T) return;
  Part acc = part_empty();
  const float4* pr = part + (int64_t)row * G;
  for (int g = lane; g < G; g += 64) {
    const float4 q = pr[g];
    acc = part_merge(acc, Part{q.x, q.y, q.z, q.w});
  }
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) {
    const Part o = shfl_xor_part(acc, s);
    acc = (lane & s) ? part_merge(o, acc) : part_merge(acc, o);
  }
  if (lane == 0) {
    if (stats) stats[row] = make_float4(acc.m, acc.R, acc.B, acc.zy);
    if (full) {
      const float L = log1pf(acc.R);
      const int32_t y = targets[row];
      const bool ok = y >= 0 && (int64_t)y < vocab_total;
      if (logp) logp[row] = ok ? (acc.zy - acc.m) - L : __builtin_nanf("");
      if (entropy) entropy[row] = L - acc.B / (1.f + acc.R);
    }
  }
}

// ======================================================== backward =======

// rowc[2t]   = {m, log1p(R), -B/(1+R), dlogp}
// rowc[2t+1] = {dentropy, bits of (y - vocab_start), 0, 0}
__global__ __launch_bounds__(kThreads) void bwd_rowprep_kernel(
    const float4* __restrict__ stats, const float* __restrict__ dlogp,
    const float* __restrict__ dent, const int32_t* __restrict__ targets, int T,
    int64_t vocab_start, float4* __restrict__ rowc) {
  const int t = blockIdx.x * kThreads + threadIdx.x;
  if (t >= T) return;
  const float4 s = stats[t];
  const float L = log1pf(s.y);
  const float Hb = -(s.z / (1.f + s.y));
  const float dl = dlogp ? dlogp[t] : 0.f;
  const float de = dent ? dent[t] : 0.f;
  const int64_t yl = (int64_t)targets[t] - vocab_start;
  const int yli = (yl < INT32_MIN || yl > INT32_MAX) ? -1 : (int)yl;
  rowc[2 * t] = make_float4(s.x, L, Hb, dl);
  rowc[2 * t + 1] = make_float4(de, __int_as_float(yli), 0.f, 0.f);
}

// G for one (T-tile, group) of the chunk, rounded to bf16 and stored twice:
// gtv[t][lg*256 + c] (row t, for dH) and gvt[lg*256 + c][t] (row v, for dW),
// both through an LDS staging tile so every global store is a full row piece.
// Rows t in [T, Tp) of gvt are written as zeros (dW reads K = Tp).
template <int BM, int WM, int WN>
__global__ __launch_bounds__(kThreads) void bwd_recompute_kernel(
    const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ weight, int T, int H,
    int V, int chunk_g0, int n_groups, int n_ttiles, const float4* __restrict__ rowc,
    uint16_t* __restrict__ gtv, int64_t ldg, uint16_t* __restrict__ gvt, int Tp) {
  using Gm = AsyncGemm<BM, GROUP, WM, WN>;
  constexpr int LDG_S = GROUP + 8;  // [t][v] staging row (bf16), 528 B
  constexpr int LDT_S = BM + 8;     // [v][t] staging row (bf16)
  constexpr int STG = (BM * LDG_S > GROUP * LDT_S ? BM * LDG_S : GROUP * LDT_S) * 2;
  constexpr int LDSB = Gm::LDS_BYTES > STG ? Gm::LDS_BYTES : STG;
  __shared__ __attribute__((aligned(16))) unsigned char lds[LDSB];
  uint16_t* stg = reinterpret_cast<uint16_t*>(lds);

  int lg, tt;
  xcd_decode(blockIdx.x, n_ttiles, lg, tt);
  if (lg >= n_groups) return;
  const int g = chunk_g0 + lg;
  const int row0 = tt * BM;
  const int col0 = g * GROUP;
  const int tid = threadIdx.x;

  Gm gm;
  gm.zero();
  gm.run(lds, hidden + (int64_t)row0 * H, H, T - row0, weight + (int64_t)col0 * H, H, V - col0, 0,
         H);

  const int lane = tid & 63;
  const int wave = wave_id();
  const int wm = wave % WM, wn = wave / WM;
  const int vlim = V - col0;
  // logit gradient in place of the logits (fp32), rounded to bf16 below
#pragma unroll
  for (int i = 0; i < Gm::MI; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int rl = wm * Gm::WTM + 16 * i + 4 * (lane >> 4) + r;
      const int t = row0 + rl;
      float4 c0 = make_float4(0.f, 0.f, 0.f, 0.f), c1 = c0;
      if (t < T) {
        c0 = rowc[2 * t];
        c1 = rowc[2 * t + 1];
      }
      const float m = c0.x, L = c0.y, Hb = c0.z, dl = c0.w, de = c1.x;
      const int yloc = __float_as_int(c1.y) - col0;
#pragma unroll
      for (int j = 0; j < Gm::NJ; ++j) {
        const int cl = wn * Gm::WTN + 16 * j + (lane & 15);
        float gv = 0.f;
        if (t < T && cl < vlim) {
          const float zd = gm.acc[i][j][r] - m;
          const float lp = zd - L;
          const float p = exp_fast(lp);
          const float onehot_term = (cl == yloc) ? -expm1f(lp) : -p;  // [v==y] - p
          gv = dl * onehot_term - de * (p * (zd + Hb));
        }
        gm.acc[i][j][r] = gv;
      }
    }
  }
  // (1) [v][t] tile -> gvt rows: each lane holds 4 consecutive t of one column
  if (gvt) {
#pragma unroll
    for (int i = 0; i < Gm::MI; ++i) {
      const int rl0 = wm * Gm::WTM + 16 * i + 4 * (lane >> 4);
#pragma unroll
      for (int j = 0; j < Gm::NJ; ++j) {
        const int cl = wn * Gm::WTN + 16 * j + (lane & 15);
        const uint32_t lo = f32_to_bf16_rne(gm.acc[i][j][0]) | (f32_to_bf16_rne(gm.acc[i][j][1]) << 16);
        const uint32_t hi = f32_to_bf16_rne(gm.acc[i][j][2]) | (f32_to_bf16_rne(gm.acc[i][j][3]) << 16);
        *reinterpret_cast<uint2*>(stg + cl * LDT_S + rl0) = make_uint2(lo, hi);
      }
    }
    __syncthreads();
    // rows of BM t values; 16 B per thread
    constexpr int TPR = BM / 8;  // threads per row
    const int tcol = (tid % TPR) * 8;
    const int t = row0 + tcol;
    if (t < Tp) {
      for (int cl = tid / TPR; cl < GROUP; cl += kThreads / TPR) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(stg + cl * LDT_S + tcol);
        *reinterpret_cast<u32x4*>(gvt + ((int64_t)lg * GROUP + cl) * Tp + t) = v;
      }
    }
    __syncthreads();
  }
  // (2) [t][v] tile -> gtv rows
  if (gtv) {
#pragma unroll
    for (int i = 0; i < Gm::MI; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int rl = wm * Gm::WTM + 16 * i + 4 * (lane >> 4) + r;
#pragma unroll
        for (int j = 0; j < Gm::NJ; ++j) {
          const int cl = wn * Gm::WTN + 16 * j + (lane & 15);
          stg[rl * LDG_S + cl] = (uint16_t)f32_to_bf16_rne(gm.acc[i][j][r]);
        }
      }
    }
    __syncthreads();
    const int c8 = (tid & 31) * 8;
    for (int rl = tid >> 5; rl < BM; rl += kThreads / 32) {
      const int t = row0 + rl;
      if (t >= T) break;
      const u32x4 v = *reinterpret_cast<const u32x4*>(stg + rl * LDG_S + c8);
      *reinterpret_cast<u32x4*>(gtv + (int64_t)t * ldg + (int64_t)lg * GROUP + c8) = v;
    }
  }
}

// hT[h][t] = hidden[t][h] for t < T, 0 for T <= t < Tp (64 x 64 tiles via LDS).
__global__ __launch_bounds__(kThreads) void transpose_hidden_kernel(
    const uint16_t* __restrict__ hidden, int T, int H, int Tp, uint16_t* __restrict__ hT) {
  __shared__ uint16_t tile[64][66];
  const int t0 = blockIdx.x * 64, h0 = blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int r = ty; r < 64; r += 4) {
    const int t = t0 + r;
    tile[r][tx] = (t < T) ? hidden[(int64_t)t * H + h0 + tx] : (uint16_t)0;
  }
  __syncthreads();
  for (int r = ty; r < 64; r += 4) {
    const int t = t0 + tx;
    if (t < Tp) hT[(int64_t)(h0 + r) * Tp + t] = tile[tx][r];
  }
}

// dW[chunk_v0 + v, h] = sum_t G[t, v] h[t, h] = sum_t gvt[v][t] hT[h][t];
// tile 256 (v) x 256 (h), K = Tp (rows t >= T are zeros in both operands).
__global__ __launch_bounds__(kThreads) void bwd_dw_kernel(
    const uint16_t* __restrict__ gvt, const uint16_t* __restrict__ hT, int Tp, int H, int V,
    int chunk_v0, int chunk_w, int n_vtiles, int n_htiles, float* __restrict__ dweight) {
  using Gm = AsyncGemm<256, 256, 2, 2>;
  __shared__ __attribute__((aligned(16))) unsigned char lds[Gm::LDS_BYTES];
  // h-tiles fastest within an XCD: one G^T tile stays hot in L2 for all of H
  int vt, ht;
  {
    const int b = blockIdx.x;
    const int xcd = b & 7, seq = b >> 3;
    vt = xcd + 8 * (seq / n_htiles);
    ht = seq % n_htiles;
  }
  if (vt >= n_vtiles) return;
  const int v0 = vt * 256, h0 = ht * 256;
  Gm gm;
  gm.zero();
  gm.run(lds, gvt + (int64_t)v0 * Tp, Tp, chunk_w - v0, hT + (int64_t)h0 * Tp, Tp, H - h0, 0, Tp);
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int wm = wave % 2, wn = wave / 2;
#pragma unroll
  for (int i = 0; i < Gm::MI; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int vl = v0 + wm * Gm::WTM + 16 * i + 4 * (lane >> 4) + r;
      const int64_t v = (int64_t)chunk_v0 + vl;
      if (vl >= chunk_w || v >= V) continue;
      float* rowp = dweight + v * H;
#pragma unroll
      for (int j = 0; j < Gm::NJ; ++j) {
        const int h = h0 + wn * Gm::WTN + 16 * j + (lane & 15);
        if (h < H) rowp[h] = gm.acc[i][j][r];
      }
    }
  }
}

// dH partial of split (split_base + si): rows t of the T-tile, columns h of
// the H-tile, v over [s_begin, s_end) of the chunk in ascending order.
template <int BM, int WM, int WN>
__global__ __launch_bounds__(kThreads) void bwd_dh_kernel(
    const uint16_t* __restrict__ gtv, int64_t ldg, const uint16_t* __restrict__ weight, int T,
    int H, int V, int chunk_v0, int split_w, int n_splits, int split_base, int n_ttiles,
    int n_htiles, float* __restrict__ part) {
  using Gm = TileGemm<BM, 256, WM, WN, false, true>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[Gm::LDS_BYTES / 2];
  // T-tiles fastest within an XCD so W[split, h-tile] is shared in L2
  int tt, rest;
  {
    const int b = blockIdx.x;
    const int xcd = b & 7, seq = b >> 3;
    rest = xcd + 8 * (seq / n_ttiles);
    tt = seq % n_ttiles;
  }
  if (rest >= n_htiles * n_splits) return;
  const int ht = rest % n_htiles;
  const int si = rest / n_htiles;
  const int row0 = tt * BM, h0 = ht * 256;
  const int s_begin = si * split_w;
  const int s_end = min(s_begin + split_w, V - chunk_v0);
  Gm gm;
  gm.zero();
  gm.run(lds, gtv + (int64_t)row0 * ldg, ldg, T - row0, weight + (int64_t)chunk_v0 * H + h0, H,
         H - h0, s_begin, s_end);
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int wm = wave % WM, wn = wave / WM;
  float* out = part + (int64_t)(split_base + si) * T * H;
#pragma unroll
  for (int i = 0; i < Gm::MI; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = row0 + wm * Gm::WTM + 16 * i + 4 * (lane >> 4) + r;
      if (t >= T) continue;
      float* rowp = out + (int64_t)t * H;
#pragma unroll
      for (int j = 0; j < Gm::NJ; ++j) {
        const int h = h0 + wn * Gm::WTN + 16 * j + (lane & 15);
        if (h < H) rowp[h] = gm.acc[i][j][r];
      }
    }
  }
}

// dH = sum_{s=0}^{S-1} part[s] in order; 4 elements per thread.
__global__ __launch_bounds__(kThreads) void bwd_dh_reduce_kernel(const float* __restrict__ part,
                                                                 int S, int64_t n, int out_f32,
                                                                 void* __restrict__ out) {
  const int64_t i4 = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * 4;
  if (i4 >= n) return;
  float4 acc = *reinterpret_cast<const float4*>(part + i4);
  for (int s = 1; s < S; ++s) {
    const float4 q = *reinterpret_cast<const float4*>(part + (int64_t)s * n + i4);
    acc.x = acc.x + q.x;
    acc.y = acc.y + q.y;
    acc.z = acc.z + q.z;
    acc.w = acc.w + q.w;
  }
  if (out_f32) {
    *reinterpret_cast<float4*>(static_cast<float*>(out) + i4) = acc;
  } else {
    const uint32_t lo = f32_to_bf16_rne(acc.x) | (f32_to_bf16_rne(acc.y) << 16);
    const uint32_t hi = f32_to_bf16_rne(acc.z) | (f32_to_bf16_rne(acc.w) << 16);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + i4) = make_uint2(lo, hi);
  }
}

__global__ __launch_bounds__(kThreads) void fill_zero_kernel(float* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

// Explicit instantiations: every launched template kernel gets its host stub
// even where the host pass would not instantiate it implicitly.
#define RLK_FWD_TILE(BM, WM, WN)                                                              \
  template __global__ void fwd_tile_kernel<BM, WM, WN>(                                       \
      const uint16_t* __restrict__, const uint16_t* __restrict__, const int32_t* __restrict__, \
      int, int, int, int64_t, int, int, float4* __restrict__);
#define RLK_RECOMPUTE(BM, WM, WN)                                                             \
  template __global__ void bwd_recompute_kernel<BM, WM, WN>(                                  \
      const uint16_t* __restrict__, const uint16_t* __restrict__, int, int, int, int, int, int, \
      const float4* __restrict__, uint16_t* __restrict__, int64_t, uint16_t* __restrict__, int);
#define RLK_DH(BM, WM, WN)                                                                     \
  template __global__ void bwd_dh_kernel<BM, WM, WN>(const uint16_t* __restrict__, int64_t,    \
                                                     const uint16_t* __restrict__, int, int, int, \
                                                     int, int, int, int, int, int,              \
                                                     float* __restrict__);
RLK_FWD_TILE(32, 1, 4)
RLK_FWD_TILE(256, 2, 2)
RLK_RECOMPUTE(32, 1, 4)
RLK_RECOMPUTE(256, 2, 2)
RLK_DH(32, 1, 4)
RLK_DH(256, 2, 2)

// ======================================================== launchers ======

static inline int cdiv(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

// Launch with the optional per-launch event timer around it.
#define RLK_LAUNCH(id, kernel, grid, st, ...)                                   \
  do {                                                                          \
    prof_before(id, st);                                                        \
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(kThreads), 0, st, __VA_ARGS__); \
    prof_after(id, st);                                                         \
  } while (0)

hipError_t launch_fwd(const FwdArgs& a, hipStream_t st) {
  const int G = cdiv(a.V, GROUP);
  const int G8 = cdiv(G, 8) * 8;
  if (a.T <= kSmallT) {
    const int nt = cdiv(a.T, 32);
    RLK_LAUNCH(K_FWD_TILE, (fwd_tile_kernel<32, 1, 4>), G8 * nt, st, a.hidden, a.weight, a.targets,
               a.T, a.H, a.V, a.vocab_start, G, nt, a.part);
  } else {
    const int nt = cdiv(a.T, 256);
    RLK_LAUNCH(K_FWD_TILE, (fwd_tile_kernel<256, 2, 2>), G8 * nt, st, a.hidden, a.weight,
               a.targets, a.T, a.H, a.V, a.vocab_start, G, nt, a.part);
  }
  RLK_LAUNCH(K_FWD_COMBINE, fwd_combine_kernel, cdiv(a.T, kThreads / 64), st, a.part, a.targets,
             a.T, G, a.vocab_total, a.full, a.logp, a.entropy, a.stats);
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdArgs& a, const BwdPlan& p, hipStream_t st) {
  const int T = a.T, H = a.H, V = a.V;
  const int Tp = (int)p.Tp;
  RLK_LAUNCH(K_BWD_ROWPREP, bwd_rowprep_kernel, cdiv(T, kThreads), st, a.stats, a.dlogp,
             a.dentropy, a.targets, T, a.vocab_start, a.rowc);
  if (a.dweight) {
    prof_before(K_BWD_TRANSPOSE, st);
    hipLaunchKernelGGL(transpose_hidden_kernel, dim3(cdiv(Tp, 64), cdiv(H, 64)), dim3(kThreads), 0,
                       st, a.hidden, T, H, Tp, a.hT);
    prof_after(K_BWD_TRANSPOSE, st);
  }
  uint16_t* gtv = a.dhidden ? a.gtv : nullptr;
  uint16_t* gvt = a.dweight ? a.gvt : nullptr;
  const bool small = T <= kSmallT;
  const int bm = small ? 32 : 256;
  const int nt = cdiv(T, bm);
  const int nht = cdiv(H, 256);
  for (int c = 0; c < p.nchunks; ++c) {
    const int s0 = c * p.splits_per_chunk;
    const int s1 = s0 + p.splits_per_chunk < p.nsplits ? s0 + p.splits_per_chunk : p.nsplits;
    const int v0 = s0 * p.split_w;  // call-local
    const int v1 = (s1 * p.split_w < V) ? s1 * p.split_w : V;
    const int width = v1 - v0;
    const int ngroups = cdiv(width, GROUP);
    const int chunk_g0 = v0 / GROUP;
    const int ng8 = cdiv(ngroups, 8) * 8;
    if (small)
      RLK_LAUNCH(K_BWD_RECOMPUTE, (bwd_recompute_kernel<32, 1, 4>), ng8 * nt, st, a.hidden,
                 a.weight, T, H, V, chunk_g0, ngroups, nt, a.rowc, gtv, p.ldg, gvt, Tp);
    else
      RLK_LAUNCH(K_BWD_RECOMPUTE, (bwd_recompute_kernel<256, 2, 2>), ng8 * nt, st, a.hidden,
                 a.weight, T, H, V, chunk_g0, ngroups, nt, a.rowc, gtv, p.ldg, gvt, Tp);
    if (a.dweight) {
      const int nvt = cdiv(width, 256);
      const int nvt8 = cdiv(nvt, 8) * 8;
      RLK_LAUNCH(K_BWD_DW, bwd_dw_kernel, nvt8 * nht, st, a.gvt, a.hT, Tp, H, V, v0,
                 ngroups * GROUP, nvt, nht, a.dweight);
    }
    if (a.dhidden) {
      const int nsp = s1 - s0;
      const int rest8 = cdiv(nht * nsp, 8) * 8;
      if (small)
        RLK_LAUNCH(K_BWD_DH, (bwd_dh_kernel<32, 1, 4>), rest8 * nt, st, a.gtv, p.ldg, a.weight, T,
                   H, V, v0, p.split_w, nsp, s0, nt, nht, a.part);
      else
        RLK_LAUNCH(K_BWD_DH, (bwd_dh_kernel<256, 2, 2>), rest8 * nt, st, a.gtv, p.ldg, a.weight,
                   T, H, V, v0, p.split_w, nsp, s0, nt, nht, a.part);
    }
  }
  if (a.dhidden) {
    const int64_t n = (int64_t)T * H;
    RLK_LAUNCH(K_BWD_DH_REDUCE, bwd_dh_reduce_kernel, cdiv(n / 4, kThreads), st, a.part,
               p.nsplits, n, a.dh_f32, a.dhidden);
  }
  return hipGetLastError();
}

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  RLK_LAUNCH(K_FILL_ZERO, fill_zero_kernel, cdiv(n, kThreads), st, p, n);
  return hipGetLastError();
}

}  // namespace rlk
