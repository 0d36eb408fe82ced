// rlk_kernels.hip — gfx950 kernels of the fused, batch-invariant linear log-prob.
//
// Forward (per call):
//   fwd_tile     one workgroup per (T-tile, vocabulary group of 256 columns):
//                bf16 MFMA logits for the tile, kept in registers; per row and
//                128-column chunk the statistics (m, R, B) by a fixed in-lane
//                and 16-lane DPP tree; the 2 chunks of the group folded left
//                to right; one (m, R, B, zy) record per (row, group) written to
//                the workspace. No T x V logits ever reach memory.
//   fwd_combine  one wave per row: the row's group records folded in a fixed
//                lane-strided order plus a fixed 64-lane tree; writes logp,
//                entropy and the row's statistics record.
// Backward (per vocabulary chunk, chunks made of whole dH splits; columns in
// the padded per-slice layout of BwdPlan, each virtual slice padded to 256):
//   bwd_recompute  logits of the chunk again (same MFMA chain as the forward,
//                  so the same bits), the logit gradient G in fp32 from the
//                  row's record and upstream gradients, RNE to bf16, staged
//                  through LDS and stored [T][chunk] coalesced.
//   bwd_dw         dW[v, :] = sum_t G[t, v] h[t, :]  (both operands read
//                  K-major through transposing LDS reads), fp32, one owner
//                  per element.
//   bwd_dh         dH partial of split s = sum_{v in s} G[t, v] W[v, :], one
//                  MFMA chain over the split in ascending v; splits start at
//                  the first row of their virtual slice, sized by the slice.
//   bwd_dh_reduce  per slice the splits' partials in order, then the slices by
//                  the fixed tree; bf16 RNE or fp32.
//   dh_merge       the same tree over fp32 dH contributions of slice calls.
// Nothing uses atomics. All per-row arithmetic is independent of the tile
// shape and the grid, so every row's outputs are identical for any T.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rlk_device.h"
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

// Statistics of one row over one wave's 128 columns (a "chunk"): the lane
// holds the row's values at columns 16 j + (lane % 16), j = 0..7. In-lane
// pairwise tree over j, then the 16-lane DPP tree. Invalid columns are -inf.
struct ChunkStats {
  float m, R, B;
};
__device__ __forceinline__ ChunkStats chunk_stats(const float (&z)[8]) {
  float mx = fmaxf(fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])),
                   fmaxf(fmaxf(z[4], z[5]), fmaxf(z[6], z[7])));
  const float m = row16_max(mx);
  int nt = 0;
  float e[8], t[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const bool tie = z[j] == m;
    const bool valid = z[j] != neg_inf();
    nt += tie ? 1 : 0;
    const float d = valid ? z[j] - m : 0.f;
    e[j] = (tie || !valid) ? 0.f : exp_fast(d);
    t[j] = e[j] * d;
  }
  const float rs = ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
  const float bs = ((t[0] + t[1]) + (t[2] + t[3])) + ((t[4] + t[5]) + (t[6] + t[7]));
  ChunkStats c;
  c.m = m;
  c.R = row16_sum(rs) + (float)(row16_sum_i(nt) - 1);
  c.B = row16_sum(bs);
  return c;
}

// Group g of the call is group g % Gs of virtual slice g / Gs: columns
// (g / Gs) Vs + 256 (g % Gs) onward, at most 256 and not past the slice.
// A persistent grid (a multiple of 8 workgroups, one per CU) walks the
// (group, T-tile) items b, b + grid, ... in xcd_decode's order, so an item
// stays on the XCD of its workgroup. The next item's first pairs are issued
// as soon as the current item's mainloop ends, and land while its chunk
// statistics are computed: the epilogue works in B's pair-1 slot, which that
// prologue leaves alone. Items whose group is past G (the padding of the
// 8-way deal) are skipped.
struct FwdItem {
  int g, row0, col0, vlim;
};
__device__ __forceinline__ FwdItem fwd_item(int it, int n_ttiles, int BM, int Gs, int Vs) {
  int g, tt;
  xcd_decode(it, n_ttiles, g, tt);
  const int lg = g % Gs;
  return FwdItem{g, tt * BM, (g / Gs) * Vs + lg * GROUP, min(GROUP, Vs - lg * GROUP)};
}

// WNT: W's loads are non-temporal, for launches with one T-tile (each W line
// is then read once, and not keeping it leaves L2 to hidden, which every item
// reads); with two or more T-tiles the second read of a line needs it kept.
template <int BM, int WM, int WN, bool WNT>
__global__ __launch_bounds__(kThreads) void fwd_tile_kernel(
    const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ weight,
    const int32_t* __restrict__ targets, int T, int H, int Vs, int Gs, int64_t vocab_start, int G,
    int n_ttiles, int n_items, float4* __restrict__ part) {
  using Gm = AsyncGemmP<BM, GROUP, WM, WN, 2, WNT>;
  static_assert(WN == 2 && Gm::WTN == 128 && Gm::NJ == 8, "one 128-column chunk per wave");
  static_assert(BM * 2 * 16 + BM * 4 + kThreads * 16 <= Gm::SLOT_B,
                "chunk records, targets and the record sink fit B's pair-1 slot");
  __shared__ __attribute__((aligned(16))) unsigned char lds[Gm::LDS_BYTES];
  float4* rec = reinterpret_cast<float4*>(lds + 2 * Gm::SLOT_A + Gm::SLOT_B);  // [BM][2 chunks]
  int* ycol = reinterpret_cast<int*>(lds + 2 * Gm::SLOT_A + Gm::SLOT_B + BM * 2 * 16);  // [BM]
  float4* sink = reinterpret_cast<float4*>(lds + 2 * Gm::SLOT_A + Gm::SLOT_B + BM * 2 * 16 +
                                           BM * 4);  // [threads], written, never read

  const int stride = gridDim.x;  // a multiple of 8: items keep their XCD
  auto next_item = [&](int it) {
    while (it < n_items && fwd_item(it, n_ttiles, BM, Gs, Vs).g >= G) it += stride;
    return it;
  };
  // target of row row0 + tid (loaded early), then its column in the
  // item's group or -1. The load's row is clamped into the batch rather than
  // predicated, so every wave issues exactly one load after the item's
  // prologue; run() may then leave it in flight at its first wait
  // (target_col ignores rows past T).
  const int tid = threadIdx.x;
  auto target_of = [&](const FwdItem& f) {
    return targets[min(f.row0 + (tid < BM ? tid : 0), T - 1)];
  };
  auto target_col = [&](const FwdItem& f, int32_t y32) {
    int yc = -1;
    if (tid < BM && f.row0 + tid < T) {
      const int64_t y = (int64_t)y32 - vocab_start - f.col0;
      if (y >= 0 && y < f.vlim) yc = (int)y;
    }
    return yc;
  };

  int it = next_item(blockIdx.x);
  if (it >= n_items) return;
  FwdItem cur = fwd_item(it, n_ttiles, BM, Gs, Vs);
  int my_yc = target_col(cur, target_of(cur));
  Gm gm;
  gm.prologue(lds, hidden + (int64_t)cur.row0 * H, H, T - cur.row0, weight + (int64_t)cur.col0 * H,
              H, cur.vlim, 0, H);
  const int lane = tid & 63;
  const int wave = wave_id();
  const int wm = wave % WM, wn = wave / WM;
  const int cbase = wn * 128;  // this wave's chunk within the group
#pragma unroll 1
  for (;;) {
    const int nit = next_item(it + stride);
    const FwdItem nxt = nit < n_items ? fwd_item(nit, n_ttiles, BM, Gs, Vs) : cur;
    int32_t ny = target_of(nxt);  // in flight during the mainloop
    gm.zero();
    // the first pair in code of its own (the young wait), then the rest
    // unrolled by k-step: with the first pair peeled, the register
    // allocator keeps every accumulator chain in its AGPRs
    gm.template run<1, true>(lds, hidden + (int64_t)cur.row0 * H, H, T - cur.row0,
                             weight + (int64_t)cur.col0 * H, H, cur.vlim, 0, H,
                             /*prefetched=*/true, /*young_pending=*/true);
    // run() ends with every load drained: the next target is settled here, so
    // the compiler's wait for it never meets the next prologue's DMA
    asm volatile("" : "+v"(ny));
    const int nyc = target_col(nxt, ny);
    if (nit < n_items)
      gm.prologue(lds, hidden + (int64_t)nxt.row0 * H, H, T - nxt.row0,
                  weight + (int64_t)nxt.col0 * H, H, nxt.vlim, 0, H);

    // chunk statistics of the current item (LDS: B's pair-1 slot only)
    if (tid < BM) ycol[tid] = my_yc;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    barrier_only();
    const int vlim = cur.vlim;
    if (cbase < vlim) {
      bool cvalid[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) cvalid[j] = cbase + 16 * j + (lane & 15) < vlim;
#pragma unroll 1
      for (int i = 0; i < Gm::MI; ++i) {
        f32x4 blk[8];
        acc_row_block<0>(gm.acc, i, blk);
        int yc[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
          yc[r] = ycol[wm * Gm::WTM + 16 * i + 4 * (lane >> 4) + r] - cbase;
        // straight-line over the four rows (no branches: rows interleave)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int rl = wm * Gm::WTM + 16 * i + 4 * (lane >> 4) + r;
          float z[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) z[j] = cvalid[j] ? blk[j][r] : neg_inf();
          const ChunkStats c = chunk_stats(z);
          // target logit: held by one lane of the 16 (if in this chunk), spread by a max
          const bool yin = yc[r] >= 0 && yc[r] < 128;
          const int jt = yc[r] >> 4;
          float zl = neg_inf();
#pragma unroll
          for (int j = 0; j < 8; ++j) zl = (j == jt) ? z[j] : zl;
          // m, R, B are the same in all 16 lanes; the lane that holds the
          // target logit (lane 0 of the 16 when the target lies elsewhere)
          // writes the record, the others a slot of their own nobody reads
          // (the streaming path spreads z_y by a max tree: the same value)
          const bool owner = (yin ? (yc[r] & 15) : 0) == (lane & 15);
          float4* dst = owner ? &rec[rl * 2 + wn] : &sink[tid];
          *dst = make_float4(c.m, c.R, c.B, yin ? zl : neg_inf());
        }
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    barrier_only();
    if (tid < BM && cur.row0 + tid < T) {
      const float4 a = rec[tid * 2];
      Part acc{a.x, a.y, a.z, a.w};
      if (128 < vlim) {
        const float4 b = rec[tid * 2 + 1];
        acc = part_merge(acc, Part{b.x, b.y, b.z, b.w});
      }
      part[(int64_t)(cur.row0 + tid) * G + cur.g] = make_float4(acc.m, acc.R, acc.B, acc.zy);
    }
    if (nit >= n_items) break;
    it = nit;
    cur = nxt;
    my_yc = nyc;
  }
  wait_vmcnt<0>();
}

// ------------------------------------------------- small-batch stream ----
//
// For T <= 64 the forward is a stream over W. A unit is 128 consecutive rows
// of one virtual slice: unit iu of slice p holds slice rows 128 iu .. (the
// half iu % 2 of group iu / 2), i.e. one wave-chunk of fwd_tile's 256-column
// group. A persistent grid of n_wg workgroups (one per CU) takes units
// b, b + n_wg, ... and runs them as ONE pipeline of stages of 32 KS k: the ring of
// NST slots keeps NST - 1 stages in flight across unit boundaries, and a
// unit's epilogue runs while the next unit's first stages land.
//
// Wave w multiplies the MI 16-row blocks of hidden by column blocks 2w and
// 2w + 1 of the unit (so a stage costs each wave 2 + MI fragment reads and
// 2 MI MFMAs, whatever T), every logit from the same MFMA chain as in
// fwd_tile (k ascending in steps of 32 from zero). At the end of a unit the
// logits pass through LDS so that each 16-lane group holds one row's 128
// columns in fwd_tile's arrangement (lane l: columns 16 j + l), and the
// record comes from the same chunk tree; the combine merges a group's two
// halves as fwd_tile does, so the bits match the large-batch path.
//
// W is read either in its natural [V, H] layout (a stage holds 128 bytes of
// each of the unit's 128 rows when H is a multiple of 128, else 64) or packed
// by pack_weight_kernel (a stage is 8 KB contiguous, already in the slot's
// LDS order), which streams from HBM at a higher rate than 128 strided
// 64-byte pieces.
constexpr int kStreamRows = 64;  // rows of hidden per launch
// Per row count (MI 16-row blocks) and k-steps per stage (KS): a stage holds
// 16 MI rows of hidden and the unit's 128 W rows, 64 KS bytes each; the
// logit buffer holds 128 columns of 16 MI rows at a stride of ZS floats
// (ZS = 4 mod 64 keeps the epilogue's reads and writes free of bank
// conflicts); the ring takes what remains.
template <int MI, int KS>
struct StreamCfg {
  static constexpr int STAGE = (16 * MI + 128) * 64 * KS;
  static constexpr int ZS = 16 * MI + 4;
  static constexpr int ZBYTES = 128 * ZS * 4;
  static constexpr int NST = (160 * 1024 - ZBYTES) / STAGE;
};

// KS = 2 (H a multiple of 128): a stage is a pair of k-steps. Hidden, and W in
// its natural layout, are staged as 128 bytes of each row, so every DMA
// request carries a whole line, the pieces of staged row r at slot
// (piece + r) mod 8 as in the tile forward; packed W is two consecutive
// packed stages, 16 KB contiguous, each in its single-step LDS order.
template <int MI, bool PACKED, int KS>
__global__ __launch_bounds__(kThreads) void fwd_stream_kernel(
    const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ weight,
    const int32_t* __restrict__ targets, int T, int H, int Vs, int Us, int P, int Gs,
    int64_t vocab_start, int n_wg, int ldp, float4* __restrict__ part) {
  static_assert(MI == 1 || MI == 2 || MI == 4, "16, 32 or 64 rows");
  static_assert(KS == 1 || KS == 2, "one k-step or a pair a stage");
  using C = StreamCfg<MI, KS>;
  constexpr int NST = C::NST, STAGE = C::STAGE, ZS = C::ZS;
  constexpr int ROWB = 64 * KS;  // bytes of a staged row
  constexpr int A_BYTES = 16 * MI * ROWB;
  constexpr int NA2 = 2 * MI;  // KS = 2: 1 KB blocks (8 rows) of hidden per stage
  static_assert(NST >= 3 && NST * STAGE + C::ZBYTES <= 160 * 1024, "ring and logits fit the LDS");
  static_assert((KS == 1 ? 3 : 6) * (NST - 2) < 64, "vmcnt range");
  __shared__ __attribute__((aligned(16))) unsigned char lds[NST * STAGE];
  __shared__ __attribute__((aligned(16))) float zbuf[128 * ZS];  // [column][row]
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int n_units = P * Us;
  const int my_units = (int)blockIdx.x < n_units ? (n_units - 1 - (int)blockIdx.x) / n_wg + 1 : 0;
  const int nsteps = H / (32 * KS);  // stages of a unit
  const int Q = my_units * nsteps;   // stages of this workgroup, all units in a row

  // targets of this lane's epilogue rows 16 i + 4 wave + lane / 16
  int yv[MI];
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    const int row = 16 * i + 4 * wave + (lane >> 4);
    yv[i] = targets[row < T ? row : 0];  // T >= 1: the loads are in flight together
  }
#pragma unroll
  for (int i = 0; i < MI; ++i) asm volatile("" ::"v"(yv[i]) : "memory");  // landed before any DMA

  const uint32_t lds0 = lds_addr(lds);
  const int drow = lane >> 2;
  const int dpiece = row_piece(lane & 3, drow);
  const i32x4 rsA = make_rsrc(hidden, (uint32_t)((T < 16 * MI ? T : 16 * MI) * H * 2));
  const bool loads_a = wave < MI;  // waves 0 .. MI-1 move one 16-row block of hidden each
  const int voffA = (16 * wave + drow) * H * 2 + 16 * dpiece;
  const int voffB0 = PACKED ? 1024 * wave + 16 * lane : (16 * wave + drow) * H * 2 + 16 * dpiece;
  const int voffB1 = PACKED ? 1024 * (wave + 4) + 16 * lane
                            : (16 * (wave + 4) + drow) * H * 2 + 16 * dpiece;
  const int sB = PACKED ? 8192 : ROWB;  // bytes between consecutive stages of a unit's B
  // KS = 2: 8-row blocks, lane -> row 8 (wave + 4 k) + lane / 8 (k = 0, 1, ... in
  // the block's vector offset, so the range check covers every row), physical
  // piece lane % 8 holding logical piece (lane % 8 - row) mod 8
  const int prow = 8 * wave + (lane >> 3);
  const int ppiece = ((lane & 7) - prow) & 7;
  const int nA2w = wave < NA2 ? (NA2 - wave + 3) / 4 : 0;  // hidden blocks of this wave
  int voffA2[2], voffB2[4];
#pragma unroll
  for (int k = 0; k < 2; ++k) voffA2[k] = (prow + 32 * k) * H * 2 + 16 * ppiece;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    voffB2[k] = PACKED ? 1024 * (wave + 4 * k) + 16 * lane : (prow + 32 * k) * H * 2 + 16 * ppiece;

  // issue state: the next stage to issue is stage iss_s of this workgroup's unit iss_u
  int iss_u = 0, iss_s = 0;
  i32x4 rsB;
  auto set_unit = [&](int i) {
    const int pu = (int)blockIdx.x + i * n_wg;
    const int p = pu / Us, iu = pu - p * Us;
    if constexpr (PACKED)
      rsB = make_rsrc(weight + (int64_t)pu * 128 * H, (uint32_t)(128 * H * 2));
    else
      rsB = make_rsrc(weight + ((int64_t)p * Vs + 128 * iu) * H,
                      (uint32_t)(min(128, Vs - 128 * iu) * H * 2));
  };
  auto issue = [&](int slot) {
    const uint32_t st = lds0 + (uint32_t)(slot * STAGE);
    if constexpr (KS == 1) {
      if (loads_a) dma16(rsA, st + 1024u * wave, voffA, 64 * iss_s);
      dma16(rsB, st + A_BYTES + 1024u * wave, voffB0, sB * iss_s);
      dma16(rsB, st + A_BYTES + 1024u * (wave + 4), voffB1, sB * iss_s);
    } else {
#pragma unroll
      for (int k = 0; k < 2; ++k)
        if (k < nA2w) dma16(rsA, st + 1024u * (wave + 4 * k), voffA2[k], ROWB * iss_s);
#pragma unroll
      for (int k = 0; k < 4; ++k)
        dma16(rsB, st + A_BYTES + 1024u * (wave + 4 * k), voffB2[k],
              (PACKED ? 16384 : ROWB) * iss_s);
    }
    if (++iss_s == nsteps) {
      iss_s = 0;
      if (++iss_u < my_units) set_unit(iss_u);
    }
  };

  if (Q > 0) set_unit(0);
  for (int q = 0; q < NST - 1 && q < Q; ++q) issue(q);

  // fragment offsets of this lane (row lane % 16 of a 16-row block) in 64-byte
  // rows (single steps, packed W) and, for k-step h, in 128-byte rows
  const int foff1 = (lane & 15) * 64 + 16 * row_slot(lane >> 4, lane & 15);
  auto foff2 = [&](int h) {
    return (lane & 15) * 128 + 16 * ((4 * h + (lane >> 4) + (lane & 15)) & 7);
  };
  f32x4 acc[MI][2];
#pragma unroll
  for (int i = 0; i < MI; ++i) acc[i][0] = acc[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  int unit = 0, s = 0;
  for (int q = 0; q < Q; ++q) {
    // this wave's DMA of stage q has landed once at most NST - 2 later stages are
    // pending (per stage: 2 W blocks, and 1 of hidden for waves < MI; with k-step
    // pairs 4 W blocks, and nA2w of hidden)
    if (q + NST - 2 >= Q)
      wait_vmcnt<0>();
    else if (KS == 1 ? loads_a : nA2w == 1)
      wait_vmcnt<(KS == 1 ? 3 : 5) * (NST - 2)>();
    else if (KS == 1 || nA2w == 0)
      wait_vmcnt<(KS == 1 ? 2 : 4) * (NST - 2)>();
    else
      wait_vmcnt<(KS == 1 ? 2 : 6) * (NST - 2)>();
    barrier_only();  // every wave's part of stage q is in; slot (q - 1) % NST is free
    if (q + NST - 1 < Q) issue((q + NST - 1) % NST);
    const unsigned char* st = lds + (q % NST) * STAGE;
#pragma unroll
    for (int h = 0; h < KS; ++h) {
      const int fa = KS == 1 ? foff1 : foff2(h);  // hidden
      // W: 16-row block 2 wave + jj of the unit at byte wb + jj wbs
      const int wb = KS == 1   ? A_BYTES + 32 * wave * 64 + foff1
                     : PACKED ? A_BYTES + 8192 * h + 32 * wave * 64 + foff1
                              : A_BYTES + 32 * wave * 128 + foff2(h);
      const int wbs = KS == 2 && !PACKED ? 16 * 128 : 16 * 64;
      const bf16x8 b0 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(st + wb));
      const bf16x8 b1 =
          __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(st + wb + wbs));
      bf16x8 af[MI];
#pragma unroll
      for (int i = 0; i < MI; ++i)
        af[i] =
            __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(st + 16 * i * ROWB + fa));
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        acc[i][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], b0, acc[i][0], 0, 0, 0);
        acc[i][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], b1, acc[i][1], 0, 0, 0);
      }
    }
    if (++s < nsteps) continue;

    // ---- unit epilogue: logits to LDS, column-major ([col][row], ZS floats a column)
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
        *reinterpret_cast<f32x4*>(&zbuf[(32 * wave + 16 * jj + (lane & 15)) * ZS + 16 * i +
                                        4 * (lane >> 4)]) = acc[i][jj];
    __syncthreads();
    const int pu = (int)blockIdx.x + unit * n_wg;
    const int p = pu / Us, iu = pu - p * Us;
    const int vlim = min(128, Vs - 128 * iu);
    const int64_t col0 = (int64_t)p * Vs + 128 * iu;  // call-relative first column
    const int u = p * 2 * Gs + iu;                   // record index (group iu / 2, half iu % 2)
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      // one row per 16-lane group: the 128 columns as fwd_tile's wave holds them
      const int row = 16 * i + 4 * wave + (lane >> 4);
      float z[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float v = zbuf[(16 * j + (lane & 15)) * ZS + row];
        z[j] = 16 * j + (lane & 15) < vlim ? v : neg_inf();
      }
      const ChunkStats c = chunk_stats(z);
      const int64_t yc = (int64_t)yv[i] - vocab_start - col0;
      const bool yin = row < T && yc >= 0 && yc < vlim;
      const int ycl = yin ? (int)yc : 0;
      const int jt = ycl >> 4;
      float zl = neg_inf();
#pragma unroll
      for (int j = 0; j < 8; ++j) zl = (j == jt) ? z[j] : zl;
      zl = (yin && (ycl & 15) == (lane & 15)) ? zl : neg_inf();
      const float zy = row16_max(zl);
      if ((lane & 15) == 0 && row < T) part[(int64_t)row * ldp + u] = make_float4(c.m, c.R, c.B, zy);
    }
    // zbuf is rewritten only after at least one more stage barrier (nsteps >= 2),
    // which every wave reaches after its reads above have returned
#pragma unroll
    for (int i = 0; i < MI; ++i) acc[i][0] = acc[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    s = 0;
    ++unit;
  }
  wait_vmcnt<0>();
}

// W rearranged for fwd_stream_kernel<PACKED>: unit pu = p Us + iu (slice p,
// slice rows 128 iu .. + 127) is 128 H elements at pu 128 H; its stage s
// (k = 32 s .. + 31) is 8 KB at s 4096 inside it, laid out exactly as a B
// slot of the ring: 16-byte piece i of 1 KB block jb holds row 16 jb + i / 4,
// k piece row_piece(i % 4, i / 4). Rows past the slice are zero.
// One thread moves one 16-byte piece: eight consecutive threads read one
// whole 128-byte line of a W row (two stages' worth of that row), a wave
// reads eight rows' lines, and its writes fill two 512-byte runs of slots.
__global__ __launch_bounds__(kThreads) void pack_weight_kernel(
    const uint16_t* __restrict__ weight, int H, int Vs, int Us, int64_t n_pieces,
    uint16_t* __restrict__ packed) {
  const int pairs = H / 64;  // 128-byte lines per W row
  for (int64_t q = (int64_t)blockIdx.x * kThreads + threadIdx.x; q < n_pieces;
       q += (int64_t)gridDim.x * kThreads) {
    const int e = (int)(q & 7);  // 16-byte piece of the line
    const int r = (int)((q >> 3) & 127);
    const int64_t rest = q >> 10;
    const int s2 = (int)(rest % pairs);
    const int64_t pu = rest / pairs;
    const int p = (int)(pu / Us), iu = (int)(pu - (int64_t)p * Us);
    const int srow = 128 * iu + r;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (srow < Vs)
      v = *reinterpret_cast<const u32x4*>(weight + ((int64_t)p * Vs + srow) * H + 64 * s2 + 8 * e);
    uint16_t* dst = packed + pu * 128 * H + (int64_t)(2 * s2 + (e >> 2)) * 4096 + 32 * r +
                    8 * row_slot(e & 3, r & 15);
    *reinterpret_cast<u32x4*>(dst) = v;
  }
}

// ==================================================== forward combine ====

__device__ __forceinline__ Part shfl_xor_part(const Part& p, int s) {
  return Part{__shfl_xor(p.m, s), __shfl_xor(p.R, s), __shfl_xor(p.B, s), __shfl_xor(p.zy, s)};
}

// Final outputs of one row from its whole-vocabulary record.
__device__ __forceinline__ void finalize_row(const Part& acc, bool target_ok, float* logp,
                                             float* entropy) {
  const float L = log1pf(acc.R);
  if (logp) *logp = target_ok ? (acc.zy - acc.m) - L : __builtin_nanf("");
  if (entropy) *entropy = L - acc.B / (1.f + acc.R);
}

// One wave per row. Each virtual slice's groups: lane j folds groups j,
// j + 64, ... of the slice in order, then a 64-lane xor tree (lower lane
// left); the P slice records then merge by the fixed tree (P = 1, 2 or 4).
// One workgroup per row; wave p folds virtual slice p: lane j merges groups
// j, j + 64, ... in order (their records loaded four at a time ahead of the
// merges), then a 64-lane xor tree with the lower lane as left operand; wave
// 0 merges the slice records by the fixed tree and finalises. With units = 2
// the records are per 128-column half (the streaming kernel) and a group's
// record is merged from its halves here, as fwd_tile merges them.
__global__ __launch_bounds__(kThreads) void fwd_combine_kernel(
    const float4* __restrict__ part, const int32_t* __restrict__ targets, int T, int G, int P,
    int Gs, int Vs, int units, int64_t vocab_total, int full, float* __restrict__ logp,
    float* __restrict__ entropy, float4* __restrict__ stats) {
  static_assert(kThreads / 64 >= kVirtualSlices, "a wave per virtual slice");
  __shared__ float4 srec[kVirtualSlices];
  const int row = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int p = wave_id();
  const float4* pr = part + (int64_t)row * G * units;
  constexpr int NB = 4;
  auto load = [&](int g, float4& a, float4& b) {
    if (units == 1) {
      a = pr[p * Gs + g];
    } else {
      a = pr[2 * (p * Gs + g)];
      if (128 < min(GROUP, Vs - g * GROUP)) b = pr[2 * (p * Gs + g) + 1];
    }
  };
  auto group_rec = [&](const float4& a, const float4& b, int g) {
    Part q{a.x, a.y, a.z, a.w};
    if (units == 2 && 128 < min(GROUP, Vs - g * GROUP)) q = part_merge(q, Part{b.x, b.y, b.z, b.w});
    return q;
  };
  if (p < P) {
    Part acc = part_empty();
    for (int g0 = lane; g0 < Gs; g0 += 64 * NB) {
      float4 ta[NB], tb[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b)
        if (g0 + 64 * b < Gs) load(g0 + 64 * b, ta[b], tb[b]);
#pragma unroll
      for (int b = 0; b < NB; ++b)
        if (g0 + 64 * b < Gs) acc = part_merge(acc, group_rec(ta[b], tb[b], g0 + 64 * b));
    }
#pragma unroll
    for (int s = 1; s < 64; s <<= 1) {
      const Part o = shfl_xor_part(acc, s);
      const bool hi = (lane & s) != 0;  // the lower lane is the left operand
      acc = part_merge(hi ? o : acc, hi ? acc : o);
    }
    if (lane == 0) srec[p] = make_float4(acc.m, acc.R, acc.B, acc.zy);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    Part rs[kVirtualSlices];
#pragma unroll
    for (int q = 0; q < kVirtualSlices; ++q) {
      const float4 v = srec[q < P ? q : 0];
      rs[q] = Part{v.x, v.y, v.z, v.w};
    }
    Part acc = rs[0];
    if (P == 2) acc = part_merge(rs[0], rs[1]);
    if (P == 4) acc = part_merge(part_merge(rs[0], rs[1]), part_merge(rs[2], rs[3]));
    if (stats) stats[row] = make_float4(acc.m, acc.R, acc.B, acc.zy);
    if (full) {
      const int32_t y = targets[row];
      finalize_row(acc, y >= 0 && (int64_t)y < vocab_total, logp ? logp + row : nullptr,
                   entropy ? entropy + row : nullptr);
    }
  }
}

// Merge of S slice records per row (slices in vocabulary order) by the fixed
// tree: a stack of subtrees of decreasing power-of-two sizes, equal
// neighbours merged left + right as records arrive, the rest folded from the
// right. One thread per row.
__global__ __launch_bounds__(kThreads) void combine_kernel(const float4* __restrict__ partials,
                                                           int S, int T, float* __restrict__ logp,
                                                           float* __restrict__ entropy,
                                                           float4* __restrict__ stats) {
  const int row = blockIdx.x * kThreads + threadIdx.x;
  if (row >= T) return;
  Part st[kCombineDepth];
  int lvl[kCombineDepth];
  int n = 0;
  for (int s = 0; s < S; ++s) {
    const float4 q = partials[(int64_t)s * T + row];
    st[n] = Part{q.x, q.y, q.z, q.w};
    lvl[n++] = 0;
    while (n >= 2 && lvl[n - 2] == lvl[n - 1]) {
      st[n - 2] = part_merge(st[n - 2], st[n - 1]);
      ++lvl[n - 2];
      --n;
    }
  }
  Part acc = st[n - 1];
  for (int i = n - 2; i >= 0; --i) acc = part_merge(st[i], acc);
  if (stats) stats[row] = make_float4(acc.m, acc.R, acc.B, acc.zy);
  finalize_row(acc, true, logp ? logp + row : nullptr, entropy ? entropy + row : nullptr);
}

// ======================================================== backward =======

// A row's constants for the logit gradient, from its whole-vocabulary
// record s = (m, R, B, z_y) and upstream gradients dl, de:
// c0 = {m, log1p(R), -B/(1+R), dl}, c1 = {de, bits of (y - vocab_start) or -1, R/(1+R), 0}.
__device__ __forceinline__ void row_constants(float4 s, float dl, float de, int32_t y,
                                              int64_t vocab_start, float4& c0, float4& c1) {
  const float L = log1pf(s.y);
  const float Hb = -(s.z / (1.f + s.y));
  const int64_t yl = (int64_t)y - vocab_start;
  const int yli = (yl < INT32_MIN || yl > INT32_MAX) ? -1 : (int)yl;
  c0 = make_float4(s.x, L, Hb, dl);
  c1 = make_float4(de, __int_as_float(yli), s.y / (1.f + s.y), 0.f);
}

// Padded column u of the backward layout: virtual slice q = u / Vs_pad,
// slice row l = u - q Vs_pad, call-local vocabulary row q Vs + l (valid while
// l < Vs).
__device__ __forceinline__ void padded_col(int u, int Vs, int Vs_pad, int& row, int& valid) {
  const int q = u / Vs_pad;
  const int l = u - q * Vs_pad;
  row = q * Vs + l;
  valid = Vs - l;
}

// G for the (T-tile, BN-column tile) items of the chunk, rounded to bf16 and
// stored as gtv[t][lt*BN + c] (rows t < T, 16-byte row pieces; the tile's
// columns past its slice's end are zeros, which covers dH's k-range at the
// end of every split; dW's tiles end on them too). Both dH and dW read G
// from there. Each element depends on its logit and its row's constants
// only, so the column width of the tile does not change a bit. Items cover
// the chunk's padded columns [u0, u0 + n_tiles BN).
// A persistent grid (a multiple of 8 workgroups; for 256-row tiles one per
// CU, for the small batch's 32-row tiles one per item) walks the items
// b, b + grid, ... in xcd_decode's order, so an item stays on the
// XCD of its workgroup. The next item's first pair is issued as soon as the
// current mainloop ends and lands while the current tile's G is formed: the
// epilogue works only in A's and B's pair-1 slots, 32 rows a round (row
// block i of both wave rows) staged as [t][v] so that the stores are whole
// 16-byte row pieces, the rounds alternating between the two slots, and the
// rows' constants (from their records and upstream gradients, loaded during
// the mainloop) beside the first round's buffer. When every wave issued all of a tile's stores, the next
// mainloop's first wait leaves them in flight.
template <int BM, int BN, int WM, int WN, bool WNT>
__global__ __launch_bounds__(kThreads) void bwd_recompute_kernel(
    const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ weight, int T, int H,
    int u0, int Vs, int Vs_pad, int n_tiles, int n_ttiles, int n_items,
    const float4* __restrict__ stats, const float* __restrict__ dlogp,
    const float* __restrict__ dent, const int32_t* __restrict__ targets, int64_t vocab_start,
    uint16_t* __restrict__ gtv, int64_t ldg) {
  using Gm = AsyncGemmP<BM, BN, WM, WN, 2, WNT>;  // WNT: W's loads non-temporal
  static_assert(WM == 2, "a round is row block i of both wave rows: 32 rows");
  constexpr int LDG_S = BN + 8;           // staged row (bf16), 16 B longer than the tile's
  constexpr int RBYTES = 32 * LDG_S * 2;  // one round
  constexpr int TPR = BN / 8;             // threads per staged row, 16 bytes each
  constexpr int RPP = kThreads / TPR;     // rows per store pass
  static_assert(kThreads % TPR == 0 && 32 % RPP == 0, "whole rows per pass, whole passes per round");
  constexpr int STORES = Gm::MI * (32 / RPP);  // store instructions of each wave for a whole tile
  constexpr bool DBL = Gm::MI > 1;             // rounds alternate between A's and B's pair-1 slots
  constexpr int OFF_A1 = Gm::SLOT_A, OFF_B1 = 2 * Gm::SLOT_A + Gm::SLOT_B;
  // row constants: two [BM] float4 arrays, row rl at slot perm(rl), which puts
  // the rows 4 apart that one read instruction takes (rows b + 4 g + r,
  // g = lane / 16) in adjacent 16-byte slots
  constexpr int OFF_TAB = OFF_A1 + (DBL ? RBYTES : 0);
  static_assert(RBYTES <= Gm::SLOT_B, "a round fits B's pair-1 slot");
  static_assert(OFF_TAB + BM * 32 <= OFF_A1 + Gm::SLOT_A, "a round and the constants fit A's");
  __shared__ __attribute__((aligned(16))) unsigned char lds[Gm::LDS_BYTES];
  float4* tab0 = reinterpret_cast<float4*>(lds + OFF_TAB);
  float4* tab1 = tab0 + BM;
  auto perm = [](int rl) { return (rl & ~15) | ((rl & 3) << 2) | ((rl >> 2) & 3); };

  struct Item {
    int row0, lg, col0, vlim;  // col0: call-local vocabulary row of the first column; vlim: valid columns
  };
  auto item_of = [&](int it) {
    int lg, tt;
    xcd_decode(it, n_ttiles, lg, tt);
    Item r;
    r.row0 = tt * BM;
    r.lg = lg;
    padded_col(u0 + lg * BN, Vs, Vs_pad, r.col0, r.vlim);
    return r;
  };
  const int stride = gridDim.x;  // a multiple of 8: items keep their XCD
  auto next_item = [&](int it) {
    for (; it < n_items; it += stride) {
      int lg, tt;
      xcd_decode(it, n_ttiles, lg, tt);
      if (lg < n_tiles) break;
    }
    return it;
  };
  const int tid = threadIdx.x;
  int it = next_item(blockIdx.x);
  if (it >= n_items) return;
  Item cur = item_of(it);
  Gm gm;
  // a tile wholly in its slice's padding (vlim <= 0) fetches no W row
  gm.prologue(lds, hidden + (int64_t)cur.row0 * H, H, T - cur.row0,
              weight + (int64_t)cur.col0 * H, H, cur.vlim, 0, H);
  const int lane = tid & 63;
  const int wave = wave_id();
  const int wm = wave % WM, wn = wave / WM;
  bool young = false;  // every wave has issued all of the previous tile's stores
#pragma unroll 1
  for (;;) {
    // this tile's rows' records and upstream gradients (thread tid: row
    // row0 + tid; rows past T take row T - 1 and are zeroed below), in
    // flight during the mainloop
    float4 rs = make_float4(0.f, 0.f, 0.f, 0.f);
    float rdl = 0.f, rde = 0.f;
    int32_t ry = 0;
    if (tid < BM) {
      const int t = cur.row0 + tid < T ? cur.row0 + tid : T - 1;
      rs = stats[t];
      if (dlogp) rdl = dlogp[t];
      if (dent) rde = dent[t];
      ry = targets[t];
    }
    gm.zero();
    gm.template run<STORES, true>(lds, hidden + (int64_t)cur.row0 * H, H, T - cur.row0,
                            weight + (int64_t)cur.col0 * H, H, cur.vlim, 0, H,
                            /*prefetched=*/true, young);
    // run() ends with every load drained: the constants are settled here, so
    // the compiler's wait for them never meets the next prologue's DMA
    asm volatile("" : "+v"(rs.x), "+v"(rs.y), "+v"(rs.z), "+v"(rs.w), "+v"(rdl), "+v"(rde),
                 "+v"(ry));
    float4 c0, c1;
    row_constants(rs, rdl, rde, ry, vocab_start, c0, c1);
    const int nit = next_item(it + stride);
    const bool more = nit < n_items;
    const Item nxt = more ? item_of(nit) : cur;
    if (more)
      gm.prologue(lds, hidden + (int64_t)nxt.row0 * H, H, T - nxt.row0,
                  weight + (int64_t)nxt.col0 * H, H, nxt.vlim, 0, H);

    // ---- G of the current tile (LDS: A's and B's pair-1 slots only)
    if (tid < BM) {
      tab0[perm(tid)] = c0;
      tab1[perm(tid)] = c1;
    }
    bool cvalid[Gm::NJ];
#pragma unroll
    for (int j = 0; j < Gm::NJ; ++j) cvalid[j] = wn * Gm::WTN + 16 * j + (lane & 15) < cur.vlim;
    const int c8 = (tid % TPR) * 8;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    barrier_only();  // the constants are in
#pragma unroll 1
    for (int i = 0; i < Gm::MI; ++i) {
      // round i's buffer last held round i - 2, which every wave read out
      // before the barrier of round i - 1
      uint16_t* stg = reinterpret_cast<uint16_t*>(lds + ((DBL && (i & 1) == 0) ? OFF_A1 : OFF_B1));
      f32x4 blk[Gm::NJ];
      acc_row_block<0>(gm.acc, i, blk);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int rl = wm * Gm::WTM + 16 * i + 4 * (lane >> 4) + r;  // tile row
        const int rr = wm * 16 + 4 * (lane >> 4) + r;                // round row
        const bool rv = cur.row0 + rl < T;
        const float4 q0 = tab0[perm(rl)];
        const float4 q1 = tab1[perm(rl)];
        const float m = q0.x, L = q0.y, Hb = q0.z, dl = q0.w, de = q1.x;
        const int yloc = __float_as_int(q1.y) - cur.col0;
        const float Rn = q1.z;  // R / (1 + R) = 1 - p at the row maximum
#pragma unroll
        for (int j = 0; j < Gm::NJ; j += 2) {
          float gv[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int cl = wn * Gm::WTN + 16 * (j + u) + (lane & 15);
            const float zd = blk[j + u][r] - m;
            const float p = exp_fast(zd - L);
            // [v == y] - p; at the target, 1 - p is exactly R/(1+R) when z_y is
            // the row maximum (zd == 0) and has no cancellation otherwise (p <= 1/2)
            const float omp = (zd == 0.f) ? Rn : 1.f - p;
            const float onehot_term = (cl == yloc) ? omp : -p;
            const float g = dl * onehot_term - de * (p * (zd + Hb));
            // zero outside the rows and columns (+0, as a select would give),
            // by a mask: written as a select, the compiler moves g's arithmetic
            // under exec-masked branches, one per element pair, and the row's
            // 8 elements no longer interleave
            const uint32_t keep = (rv && cvalid[j + u]) ? 0xFFFFFFFFu : 0u;
            gv[u] = __uint_as_float(__float_as_uint(g) & keep);
          }
          const uint32_t pk = pack_bf16x2(gv[0], gv[1]);
          const int cl0 = wn * Gm::WTN + 16 * j + (lane & 15);
          stg[rr * LDG_S + cl0] = (uint16_t)pk;
          stg[rr * LDG_S + cl0 + 16] = (uint16_t)(pk >> 16);
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      barrier_only();
      // the round's rows: round row k is tile row (k / 16) WTM + 16 i + k % 16
#pragma unroll
      for (int k0 = 0; k0 < 32; k0 += RPP) {
        const int k = k0 + tid / TPR;
        const int t = cur.row0 + (k >> 4) * Gm::WTM + 16 * i + (k & 15);
        if (t < T) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(stg + k * LDG_S + c8);
          *reinterpret_cast<u32x4*>(gtv + (int64_t)t * ldg + (int64_t)cur.lg * BN + c8) = v;
        }
      }
    }
    young = cur.row0 + BM <= T;
    if (!more) break;
    it = nit;
    cur = nxt;
  }
  wait_vmcnt<0>();
}

// dW[chunk_v0 + v, h] = sum_t G[t, v] h[t, h], read straight from gtv [t][v]
// and hidden [t][h] (both K-major), tile 256 (v) x kDwBN (h), K = t over
// [0, Tp) with rows t >= T reading as zero.
// With K as short as one batch, the tile's fp32 output takes about as long
// to write as its MFMAs take to run. The tile is sized for two workgroups
// per CU (3-slot ring: 72 KB of LDS, 128 accumulators per lane) so that one
// can compute while the other writes, and the stores are non-temporal. The
// h-tiles are split into groups of at most 16, one group per set of XCDs,
// and the XCDs of a set split the v-tiles: an XCD keeps its 16 hidden column
// slices in L2 (2 MB at T = 512, half of it) and its ~64 resident
// workgroups share a few G column slices, so the operands stay in L2 while
// the output streams past; G is read from memory once per set. (At H = 4096
// and T = 512: 2 sets read 0.34 GB a launch, 4 sets of 8 h-tiles 0.64 GB, in
// the same time; 1 set, whose 4 MB of hidden does not stay in L2, 1.94 GB.)
DwMap dw_map(int n_vtiles, int n_htiles) {
  DwMap m;
  const int need = (n_htiles + 15) / 16;
  m.groups = need <= 1 ? 1 : need <= 2 ? 2 : need <= 4 ? 4 : 8;
  m.h_per_group = (n_htiles + m.groups - 1) / m.groups;
  m.v_per_xcd = (n_vtiles + 8 / m.groups - 1) / (8 / m.groups);
  m.per_xcd = m.v_per_xcd * m.h_per_group;
  return m;
}

// One dW tile (v-tile vt, h-tile ht) of the chunk: G columns vt 256 .. + 255
// of the buffer (padded columns u0 + vt 256 ..), dW rows from the call-local
// vocabulary row of its first column; lds holds DwGemm::LDS_BYTES.
using DwGemm = AsyncGemmKK<256, kDwBN, 2, 2, 3>;
template <bool PAD>
__device__ __forceinline__ void dw_tile(unsigned char* lds, const uint16_t* __restrict__ gtv,
                                        int64_t ldg, const uint16_t* __restrict__ hidden, int T,
                                        int Tp, int H, int u0, int Vs, int Vs_pad, int vt, int ht,
                                        float* __restrict__ dweight) {
  using Gm = DwGemm;
  const int v0 = vt * 256, h0 = ht * kDwBN;
  Gm gm;
  gm.zero();
  gm.template run<PAD>(lds, gtv + v0, ldg, T, 256, hidden + h0, H, T, min(kDwBN, H - h0), 0, Tp);
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int wm = wave % 2, wn = wave / 2;
  // The output leaves through the freed ring, 128 rows at a time: the two
  // waves that own the rows write their accumulators to LDS, then every wave
  // stores whole rows, 32 lanes x 16 bytes covering one 512-byte row segment,
  // so each write request carries full lines (written from the accumulator
  // layout, a store instruction carries 64-byte pieces of four rows).
  static_assert(Gm::WTM == 128 && kDwBN == 128, "one half-tile of rows per wave row");
  constexpr int ZS = kDwBN + 4;  // floats per staged row (conflict-free writes)
  static_assert(128 * ZS * 4 <= Gm::LDS_BYTES, "half a tile fits the ring");
  float* stage = reinterpret_cast<float*>(lds);
  int vrow0, vlim;  // call-local vocabulary row of the tile's first row; valid rows
  padded_col(u0 + v0, Vs, Vs_pad, vrow0, vlim);
  const int hcols = min(kDwBN, H - h0);  // a multiple of 64
  const int c4 = 4 * (lane & 31);        // column of this lane's 16 bytes
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if (wm == half) {
#pragma unroll
      for (int i = 0; i < Gm::MI; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * i + 4 * (lane >> 4) + r;
#pragma unroll
          for (int j = 0; j < Gm::NJ; ++j)
            stage[row * ZS + wn * Gm::WTN + 16 * j + (lane & 15)] = gm.acc[i][j][r];
        }
    }
    __syncthreads();
    // wave w stores rows 2 k + lane / 32 for k = w, w + 4, ...
#pragma unroll 4
    for (int k = wave; k < 64; k += 4) {
      const int row = 2 * k + (lane >> 5);
      const int vl = 128 * half + row;
      if (vl < vlim && c4 < hcols) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(stage + row * ZS + c4);
        __builtin_nontemporal_store(
            v, reinterpret_cast<f32x4*>(dweight + (int64_t)(vrow0 + vl) * H + h0 + c4));
      }
    }
    __syncthreads();
  }
}

// (v-tile, h-tile) of the seq-th tile of XCD xcd under `map` (ht >= n_htiles
// or vt >= n_vtiles: no tile).
__device__ __forceinline__ void dw_tile_of(const DwMap& map, int xcd, int seq, int& vt, int& ht) {
  ht = (xcd % map.groups) * map.h_per_group + seq % map.h_per_group;
  vt = (xcd / map.groups) * map.v_per_xcd + seq / map.h_per_group;
}

// PAD: the mainloop's padded refills, for K of 3 steps or more
template <bool PAD>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void
bwd_dw_kernel(const uint16_t* __restrict__ gtv, int64_t ldg, const uint16_t* __restrict__ hidden,
              int T, int Tp, int H, int u0, int Vs, int Vs_pad, int n_vtiles, int n_htiles,
              DwMap map, float* __restrict__ dweight) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[DwGemm::LDS_BYTES];
  const int seq = blockIdx.x >> 3;
  if (seq >= map.per_xcd) return;
  int vt, ht;
  dw_tile_of(map, blockIdx.x & 7, seq, vt, ht);
  if (ht >= n_htiles || vt >= n_vtiles) return;
  dw_tile<PAD>(lds, gtv, ldg, hidden, T, Tp, H, u0, Vs, Vs_pad, vt, ht, dweight);
}

// dH partials of split s (the kernel is compiled in rlk_dh.hip, on its own
// so that its translation unit can take a machine-scheduler strategy of its
// own).
template <int BM, int BN, int WM, int WN>
__global__ void bwd_dh_kernel(const uint16_t* __restrict__ gtv, int64_t ldg,
                              const uint16_t* __restrict__ weight, int T, int H, int u0,
                              SplitMap sm, int n_splits, int split_base, int n_ttiles,
                              int n_htiles, int per_xcd, float* __restrict__ part);

__device__ __forceinline__ float4 add4(const float4& a, const float4& b) {
  return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}

// Sum of S values by the fixed merge tree of the slice records: a stack of
// subtrees of decreasing power-of-two sizes, equal neighbours added left +
// right as values arrive, the rest folded from the right. S = 2 gives
// v0 + v1, S = 4 gives (v0 + v1) + (v2 + v3). next(i) yields value i.
template <class Next>
__device__ __forceinline__ float4 tree_sum(int S, Next next) {
  float4 st[kCombineDepth];
  int lvl[kCombineDepth];
  int n = 0;
  for (int i = 0; i < S; ++i) {
    st[n] = next(i);
    lvl[n++] = 0;
    while (n >= 2 && lvl[n - 2] == lvl[n - 1]) {
      st[n - 2] = add4(st[n - 2], st[n - 1]);
      ++lvl[n - 2];
      --n;
    }
  }
  float4 acc = st[n - 1];
  for (int i = n - 2; i >= 0; --i) acc = add4(st[i], acc);
  return acc;
}

__device__ __forceinline__ void store_dh4(void* out, int64_t i4, int out_f32, const float4& v) {
  if (out_f32) {
    *reinterpret_cast<float4*>(static_cast<float*>(out) + i4) = v;
  } else {
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + i4) =
        make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
  }
}

// dH of the call: per virtual slice q its n_sub split partials in order
// (part[q n_sub] + part[q n_sub + 1] + ...), then the P (1, 2 or 4) slice
// sums by the fixed tree; 4 elements per thread.
__global__ __launch_bounds__(kThreads) void bwd_dh_reduce_kernel(const float* __restrict__ part,
                                                                 int P, int n_sub, int64_t n,
                                                                 int out_f32,
                                                                 void* __restrict__ out) {
  const int64_t i4 = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * 4;
  if (i4 >= n) return;
  auto slice_sum = [&](int q) {
    const float* p = part + (int64_t)q * n_sub * n + i4;
    float4 a = *reinterpret_cast<const float4*>(p);
    for (int j = 1; j < n_sub; ++j) a = add4(a, *reinterpret_cast<const float4*>(p + j * n));
    return a;
  };
  // tree_sum's expression for P = 1, 2, 4, written out (no stack)
  float4 acc;
  if (P == 4)
    acc = add4(add4(slice_sum(0), slice_sum(1)), add4(slice_sum(2), slice_sum(3)));
  else if (P == 2)
    acc = add4(slice_sum(0), slice_sum(1));
  else
    acc = slice_sum(0);
  store_dh4(out, i4, out_f32, acc);
}

// Merge of S fp32 dH contributions of slice calls (slices in vocabulary
// order) by the same tree; 4 elements per thread.
__global__ __launch_bounds__(kThreads) void dh_merge_kernel(const float* __restrict__ parts, int S,
                                                            int64_t n, int out_f32,
                                                            void* __restrict__ out) {
  const int64_t i4 = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * 4;
  if (i4 >= n) return;
  const float4 acc = tree_sum(S, [&](int s) {
    return *reinterpret_cast<const float4*>(parts + (int64_t)s * n + i4);
  });
  store_dh4(out, i4, out_f32, acc);
}

__global__ __launch_bounds__(kThreads) void fill_zero_kernel(float* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

// Explicit instantiations: every launched template kernel gets its host stub
// even where the host pass would not instantiate it implicitly.
#define RLK_FWD_TILE(BM, WM, WN, WNT)                                                         \
  template __global__ void fwd_tile_kernel<BM, WM, WN, WNT>(                                  \
      const uint16_t* __restrict__, const uint16_t* __restrict__, const int32_t* __restrict__, \
      int, int, int, int, int64_t, int, int, int, float4* __restrict__);
#define RLK_RECOMPUTE(BM, BN, WM, WN, WNT)                                                     \
  template __global__ void bwd_recompute_kernel<BM, BN, WM, WN, WNT>(                          \
      const uint16_t* __restrict__, const uint16_t* __restrict__, int, int, int, int, int, int, \
      int, int, const float4* __restrict__, const float* __restrict__, const float* __restrict__, \
      const int32_t* __restrict__, int64_t, uint16_t* __restrict__, int64_t);
#define RLK_DW(PAD)                                                                            \
  template __global__ void bwd_dw_kernel<PAD>(const uint16_t* __restrict__, int64_t,           \
                                              const uint16_t* __restrict__, int, int, int, int, \
                                              int, int, int, int, DwMap, float* __restrict__);
RLK_DW(false)
RLK_DW(true)
RLK_FWD_TILE(256, 2, 2, false)
RLK_FWD_TILE(256, 2, 2, true)
RLK_RECOMPUTE(32, 128, 2, 2, false)
RLK_RECOMPUTE(256, 256, 2, 2, false)
RLK_RECOMPUTE(256, 256, 2, 2, true)

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
  const FwdSlicing& sl = a.slicing;
  const int G = sl.G;
  int units = 1;
  if (a.packed || a.T <= kSmallT) {
    // persistent stream over 128-row units, 64 rows of hidden per launch
    units = 2;
    const int Us = cdiv(sl.Vs, 128);
    const int n_units = sl.P * Us;
    const int n_cu = a.n_cu > 0 ? a.n_cu : 256;
    const int grid = n_cu < n_units ? n_cu : n_units;
    for (int r0 = 0; r0 < a.T; r0 += kStreamRows) {
      const int rows = a.T - r0 < kStreamRows ? a.T - r0 : kStreamRows;
      const uint16_t* h = a.hidden + (int64_t)r0 * a.H;
      const int32_t* y = a.targets + r0;
      float4* pr = a.part + (int64_t)r0 * 2 * G;
#define RLK_STREAM(MI, PK, KS)                                                                 \
  RLK_LAUNCH(K_FWD_STREAM, (fwd_stream_kernel<MI, PK, KS>), grid, st, h, a.weight, y,          \
             rows, a.H, sl.Vs, Us, sl.P, sl.Gs, a.vocab_start, grid, 2 * G, pr)
      if (a.packed && a.H % 128 == 0) {  // k-step pairs: at least two stages a unit
        if (rows <= 16) RLK_STREAM(1, true, 2);
        else if (rows <= 32) RLK_STREAM(2, true, 2);
        else RLK_STREAM(4, true, 2);
      } else if (a.packed) {
        if (rows <= 16) RLK_STREAM(1, true, 1);
        else if (rows <= 32) RLK_STREAM(2, true, 1);
        else RLK_STREAM(4, true, 1);
      } else if (a.H % 128 == 0) {  // k-step pairs: at least two stages a unit
        if (rows <= 16) RLK_STREAM(1, false, 2);
        else if (rows <= 32) RLK_STREAM(2, false, 2);
        else RLK_STREAM(4, false, 2);
      } else {
        if (rows <= 16) RLK_STREAM(1, false, 1);
        else if (rows <= 32) RLK_STREAM(2, false, 1);
        else RLK_STREAM(4, false, 1);
      }
#undef RLK_STREAM
    }
  } else {
    const int nt = cdiv(a.T, 256);
    const int n_items = cdiv(G, 8) * 8 * nt;
    const int n_cu = a.n_cu > 0 ? a.n_cu : 256;
    const int grid = min(cdiv(n_cu, 8) * 8, n_items);  // a multiple of 8
    if (nt == 1)
      RLK_LAUNCH(K_FWD_TILE, (fwd_tile_kernel<256, 2, 2, true>), grid, st, a.hidden, a.weight,
                 a.targets, a.T, a.H, sl.Vs, sl.Gs, a.vocab_start, G, nt, n_items, a.part);
    else
      RLK_LAUNCH(K_FWD_TILE, (fwd_tile_kernel<256, 2, 2, false>), grid, st, a.hidden, a.weight,
                 a.targets, a.T, a.H, sl.Vs, sl.Gs, a.vocab_start, G, nt, n_items, a.part);
  }
  RLK_LAUNCH(K_FWD_COMBINE, fwd_combine_kernel, a.T, st, a.part, a.targets,
             a.T, G, sl.P, sl.Gs, sl.Vs, units, a.vocab_total, a.full, a.logp, a.entropy, a.stats);
  return hipGetLastError();
}

hipError_t launch_pack(const uint16_t* weight, int H, const FwdSlicing& sl, uint16_t* packed,
                       hipStream_t st) {
  const int Us = cdiv(sl.Vs, 128);
  const int64_t n_pieces = (int64_t)sl.P * Us * 16 * H;
  const int64_t want = (n_pieces + kThreads - 1) / kThreads;
  const int grid = (int)(want < 16384 ? want : 16384);
  RLK_LAUNCH(K_PACK, pack_weight_kernel, grid, st, weight, H, sl.Vs, Us, n_pieces, packed);
  return hipGetLastError();
}

hipError_t launch_combine(const float4* partials, int S, int T, float* logp, float* entropy,
                          float4* stats, hipStream_t st) {
  RLK_LAUNCH(K_COMBINE, combine_kernel, cdiv(T, kThreads), st, partials, S, T, logp, entropy,
             stats);
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdArgs& a, const BwdPlan& p, hipStream_t st) {
  const int T = a.T, H = a.H;
  const int Tp = (int)p.Tp;
  const bool small = T <= kSmallT;
  const int bm = small ? 32 : 256;
  // persistent recompute: a multiple of 8 workgroups, one per CU for 256-row tiles
  const int grid_cap = cdiv(a.n_cu > 0 ? a.n_cu : 256, 8) * 8;
  const int nt = cdiv(T, bm);
  const int nht = cdiv(H, 256);
  const SplitMap sm{p.Vs, p.Vs_pad, p.n_sub, p.split_w};
  for (int c = 0; c < p.nchunks; ++c) {
    const int s0 = c * p.splits_per_chunk;
    const int s1 = s0 + p.splits_per_chunk < p.nsplits ? s0 + p.splits_per_chunk : p.nsplits;
    const int u0 = p.u_begin(s0);
    const int width = p.u_end(s1 - 1) - u0;  // padded columns of the chunk (a multiple of 256)
    if (small) {
      // 128-column tiles: the W stream of a small batch splits over twice as
      // many workgroups, so the last round is fuller
      constexpr int BN = 128;
      const int ntl = width / BN;
      const int n_items = cdiv(ntl, 8) * 8 * nt;
      // one item per workgroup (up to four resident per CU with 40 KB of LDS
      // each): for these short tiles that beats a persistent walk
      RLK_LAUNCH(K_BWD_RECOMPUTE, (bwd_recompute_kernel<32, BN, 2, 2, false>), n_items,
                 st, a.hidden, a.weight, T, H, u0, p.Vs, p.Vs_pad, ntl, nt, n_items, a.stats,
                 a.dlogp, a.dentropy, a.targets, a.vocab_start, a.gtv, p.ldg);
    } else {
      const int ntl = width / 256;
      const int n_items = cdiv(ntl, 8) * 8 * nt;
      // the chunk's G stays in the Infinity Cache for dW and dH when it fits
      // with room to spare and the recompute's W stream does not evict it
      const bool wnt = size_t(p.Tp) * size_t(width) * 2 <= kGResidentBytes;
      if (wnt)
        RLK_LAUNCH(K_BWD_RECOMPUTE, (bwd_recompute_kernel<256, 256, 2, 2, true>),
                   min(grid_cap, n_items), st, a.hidden, a.weight, T, H, u0, p.Vs, p.Vs_pad, ntl,
                   nt, n_items, a.stats, a.dlogp, a.dentropy, a.targets, a.vocab_start, a.gtv,
                   p.ldg);
      else
        RLK_LAUNCH(K_BWD_RECOMPUTE, (bwd_recompute_kernel<256, 256, 2, 2, false>),
                   min(grid_cap, n_items), st, a.hidden, a.weight, T, H, u0, p.Vs, p.Vs_pad, ntl,
                   nt, n_items, a.stats, a.dlogp, a.dentropy, a.targets, a.vocab_start, a.gtv,
                   p.ldg);
    }
    const int nvt = width / 256;
    const int nhw = cdiv(H, kDwBN);
    const int nsp = s1 - s0;
    if (a.dweight) {
      const DwMap map = dw_map(nvt, nhw);
      if (Tp > 64)
        RLK_LAUNCH(K_BWD_DW, bwd_dw_kernel<true>, 8 * map.per_xcd, st, a.gtv, p.ldg, a.hidden, T,
                   Tp, H, u0, p.Vs, p.Vs_pad, nvt, nhw, map, a.dweight);
      else
        RLK_LAUNCH(K_BWD_DW, bwd_dw_kernel<false>, 8 * map.per_xcd, st, a.gtv, p.ldg, a.hidden, T,
                   Tp, H, u0, p.Vs, p.Vs_pad, nvt, nhw, map, a.dweight);
    }
    if (a.dhidden) {
      if (small) {
        const int nh = cdiv(H, 128);
        const int per = cdiv(nt * nh * nsp, 8);
        RLK_LAUNCH(K_BWD_DH, (bwd_dh_kernel<32, 128, 1, 4>), 8 * per, st, a.gtv, p.ldg, a.weight,
                   T, H, u0, sm, nsp, s0, nt, nh, per, a.part);
      } else {
        const int per = cdiv(nt * nht * nsp, 8);
        RLK_LAUNCH(K_BWD_DH, (bwd_dh_kernel<256, 256, 2, 2>), 8 * per, st, a.gtv, p.ldg, a.weight,
                   T, H, u0, sm, nsp, s0, nt, nht, per, a.part);
      }
    }
  }
  if (a.dhidden) {
    const int64_t n = (int64_t)T * H;
    RLK_LAUNCH(K_BWD_DH_REDUCE, bwd_dh_reduce_kernel, cdiv(n / 4, kThreads), st, a.part, p.P,
               p.n_sub, n, a.dh_f32, a.dhidden);
  }
  return hipGetLastError();
}

hipError_t launch_dh_merge(const float* parts, int S, int64_t n, int out_f32, void* out,
                           hipStream_t st) {
  RLK_LAUNCH(K_DH_MERGE, dh_merge_kernel, cdiv(n / 4, kThreads), st, parts, S, n, out_f32, out);
  return hipGetLastError();
}

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  RLK_LAUNCH(K_FILL_ZERO, fill_zero_kernel, cdiv(n, kThreads), st, p, n);
  return hipGetLastError();
}

}  // namespace rlk
