// rlk_lora_fwd.hip — the LoRA forward's product tile (x W^T, then the
// adapter term or the split partial), in a translation unit of its own: the
// library's build script compiles it with the machine scheduler's
// iterative-ILP strategy, which orders the same instructions so that the
// tile streams W faster; the other LoRA kernels keep the default. The
// arithmetic, and so every bit, is the source's.
#include "rlk_lora_common.h"

namespace rlk {

// y tile (64 tokens x BN outputs): x W^T on the MFMA mainloop, then + s u B^T.
// With S > 1 splits of K the tile covers K split ks and writes its fp32
// partial to part[ks][t][n] instead (lora_fwd_reduce_kernel finishes y).
// Workgroups past the tiles (n_ttiles * n_ntiles * S of them) run the job ju
// (the rows' codes u, with S > 1 only).
template <int BN>
__global__ __launch_bounds__(kThreads) void lora_fwd_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ W, const float* __restrict__ u,
    const uint16_t* __restrict__ B, int T, int K, int N, int r, float scale, int n_ttiles,
    int n_ntiles, int S, uint16_t* __restrict__ y, float* __restrict__ part, RowdotJob ju) {
  using Gm = LoraFwdGemm<BN>;
  __shared__ __attribute__((aligned(16))) unsigned char lds[Gm::LDS_BYTES];
  const int n_main = n_ttiles * n_ntiles * S;
  if ((int)blockIdx.x >= n_main) {
    rowdot_wave<true>(ju.P, ju.Q, T, ju.L, r, ju.out,
                      ((int)blockIdx.x - n_main) * (kThreads / 64) + wave_id());
    return;
  }
  const int tt = (int)blockIdx.x % n_ttiles, rest = (int)blockIdx.x / n_ttiles;
  const int nt = rest % n_ntiles, ks = rest / n_ntiles;
  const int row0 = tt * kLoraBM, col0 = nt * BN;
  const int Ks = K / S;
  Gm gm;
  gm.zero();
  // the pair's k-steps unrolled (no branch per row block; same MFMA chain)
  gm.template run<0, true>(lds, x + (int64_t)row0 * K, K, T - row0, W + (int64_t)col0 * K, K,
                           N - col0, ks * Ks, (ks + 1) * Ks);
  if (S == 1) {
    // run() ends on a barrier: the ring is free. B's column n holds B[n][0..r-1].
    lora_epilogue<BN>(gm, lds, u, B, r, 1, T, N, r, scale, row0, col0, y, N);
    return;
  }
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int wm = wave % 2, wn = wave / 2;
  float* out = part + (int64_t)ks * T * N;
#pragma unroll
  for (int i = 0; i < Gm::MI; ++i)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int row = row0 + wm * Gm::WTM + 16 * i + 4 * (lane >> 4) + rr;
#pragma unroll
      for (int jn = 0; jn < Gm::NJ; ++jn) {
        const int col = col0 + wn * Gm::WTN + 16 * jn + (lane & 15);
        if (row < T && col < N) out[(int64_t)row * N + col] = gm.acc[i][jn][rr];
      }
    }
}

template __global__ void lora_fwd_kernel<kLoraBN>(const uint16_t* __restrict__,
                                                  const uint16_t* __restrict__,
                                                  const float* __restrict__,
                                                  const uint16_t* __restrict__, int, int, int,
                                                  int, float, int, int, int,
                                                  uint16_t* __restrict__, float* __restrict__,
                                                  RowdotJob);
template __global__ void lora_fwd_kernel<kLoraBNm>(const uint16_t* __restrict__,
                                                   const uint16_t* __restrict__,
                                                   const float* __restrict__,
                                                   const uint16_t* __restrict__, int, int, int,
                                                   int, float, int, int, int,
                                                   uint16_t* __restrict__, float* __restrict__,
                                                   RowdotJob);
template __global__ void lora_fwd_kernel<kLoraBNs>(const uint16_t* __restrict__,
                                                   const uint16_t* __restrict__,
                                                   const float* __restrict__,
                                                   const uint16_t* __restrict__, int, int, int,
                                                   int, float, int, int, int,
                                                   uint16_t* __restrict__, float* __restrict__,
                                                   RowdotJob);

}  // namespace rlk
