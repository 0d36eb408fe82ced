// dH partials of the backward: dH[t][h] = sum over the split's vocabulary
// columns v of G[t][v] W[v][h], one fp32 partial per split (bwd_dh_reduce in
// rlk_kernels.hip adds them in the fixed order). The arithmetic is described
// with dh_item below; the host launches bwd_dh_kernel from rlk_kernels.hip.
// This translation unit is built with the machine scheduler's iterative-ILP
// strategy (the library's build script passes it for this file alone): it
// orders the same instructions of the KN mainloop differently, and the
// results are the same bits.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rlk_device.h"
#include "rlk_internal.h"

namespace rlk {

// dH partial of split s (of the call): rows t of the T-tile, columns h of the
// H-tile, v over the split's columns in ascending order, one MFMA chain from
// the split's first column (its G columns start at u_begin(s) - u0 in the
// chunk buffer; its W rows at the slice's first row plus its offset). The
// span is rounded up to whole MFMA steps: the G columns past the split's end
// there are its slice's zero padding (or the next split's columns, at
// multiples of 256 no step overruns) and the W rows past it read as zero.
// Work items (t-tile fastest, then h-tile, then split) are dealt to the 8
// XCDs in contiguous runs, so one split's G rows and W rows are fetched into
// one XCD's L2 and reused there.
// The MFMA is v_mfma_f32_32x32x16_bf16 (one wave per SIMD issues it at the
// full matrix-core rate); every dH path uses it, so the split partials have
// the same bits whatever the tile.
template <int BM, int BN, int WM, int WN, int NSTG>
using DhGemm = AsyncGemmKN<BM, BN, WM, WN, NSTG, true>;

template <int BM, int BN, int WM, int WN, int NSTG>
__device__ __forceinline__ void dh_item(unsigned char* lds, const uint16_t* __restrict__ gtv,
                                        int64_t ldg, const uint16_t* __restrict__ weight, int T,
                                        int H, int u0, SplitMap sm, int tt, int ht, int s,
                                        float* __restrict__ part) {
  using Gm = DhGemm<BM, BN, WM, WN, NSTG>;
  const int row0 = tt * BM, h0 = ht * BN;
  const int q = s / sm.n_sub, j = s - q * sm.n_sub;
  const int a_col = q * sm.Vs_pad + j * sm.split_w - u0;  // chunk buffer column
  const int w_row = q * sm.Vs + j * sm.split_w;            // call-local W row
  const int len = min(sm.split_w, sm.Vs - j * sm.split_w);
  Gm gm;
  gm.zero();
  gm.run(lds, gtv + (int64_t)row0 * ldg + a_col, ldg, T - row0, weight + (int64_t)w_row * H + h0,
         H, len, min(BN, H - h0), 0, (len + 31) & ~31);
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int wm = wave % WM, wn = wave / WM;
  // a 32-column block is whole or absent (H is a multiple of 64): wave-uniform test
  const int hb = h0 + wn * Gm::WTN;
  float* const out = part + (int64_t)s * T * H + hb + (lane & 31);
  // accumulator element e of block (i, j): row 32 i + 8 (e / 4) + 4 (lane / 32) + e % 4,
  // column 32 j + lane % 32 (each store: 32 lanes x 4 bytes of one row)
#pragma unroll
  for (int i = 0; i < Gm::MI; ++i) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int t = row0 + wm * Gm::WTM + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
      if (t >= T) continue;
      float* rowp = out + (int64_t)t * H;
#pragma unroll
      for (int j = 0; j < Gm::NJ; ++j)
        if (hb + 32 * j < H) rowp[32 * j] = gm.acc[i][j][e];
    }
  }
}

template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(kThreads) void bwd_dh_kernel(
    const uint16_t* __restrict__ gtv, int64_t ldg, const uint16_t* __restrict__ weight, int T,
    int H, int u0, SplitMap sm, int n_splits, int split_base, int n_ttiles, int n_htiles,
    int per_xcd, float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[DhGemm<BM, BN, WM, WN, 4>::LDS_BYTES];
  const int seq = blockIdx.x >> 3;
  if (seq >= per_xcd) return;
  const int w = (blockIdx.x & 7) * per_xcd + seq;
  if (w >= n_ttiles * n_htiles * n_splits) return;
  const int tt = w % n_ttiles;
  const int ht = (w / n_ttiles) % n_htiles;
  const int si = w / (n_ttiles * n_htiles);
  dh_item<BM, BN, WM, WN, 4>(lds, gtv, ldg, weight, T, H, u0, sm, tt, ht, split_base + si, part);
}

// Explicit instantiations: the launchers in rlk_kernels.hip reference these.
#define RLK_DH(BM, BN, WM, WN)                                                                \
  template __global__ void bwd_dh_kernel<BM, BN, WM, WN>(                                       \
      const uint16_t* __restrict__, int64_t, const uint16_t* __restrict__, int, int, int, SplitMap, \
      int, int, int, int, int, float* __restrict__);
RLK_DH(32, 128, 1, 4)
RLK_DH(256, 256, 2, 2)

}  // namespace rlk
