// rlk_lora_common.h — pieces of the LoRA linear shared by rlk_lora.hip and
// rlk_lora_fwd.hip: the tile sizes, the forward's mainloop, the rank-r code
// waves and the adapter epilogue of a tile.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rlk_device.h"
#include "rlk_internal.h"

namespace rlk {

constexpr int kLoraBM = 64;    // rows (tokens) per tile
constexpr int kLoraBN = 128;   // output columns per tile
constexpr int kLoraBNm = 64;   // output columns per tile when wide tiles leave CUs idle
constexpr int kLoraBNs = 32;   // ... and when 64-column ones still do
constexpr int kLoraMaxRank = 64;
template <int BN>
using LoraFwdGemm = AsyncGemmP<kLoraBM, BN, 2, 2>;
using LoraDxGemm = AsyncGemmKN<kLoraBM, kLoraBN, 2, 2, 4>;
static_assert((kLoraBM + kLoraBN) * kLoraMaxRank * 4 <= LoraFwdGemm<kLoraBN>::LDS_BYTES &&
                  (kLoraBM + kLoraBNm) * kLoraMaxRank * 4 <= LoraFwdGemm<kLoraBNm>::LDS_BYTES &&
                  (kLoraBM + kLoraBNs) * kLoraMaxRank * 4 <= LoraFwdGemm<kLoraBNs>::LDS_BYTES &&
                  (kLoraBM + kLoraBN) * kLoraMaxRank * 4 <= LoraDxGemm::LDS_BYTES,
              "the adapter operands of a tile fit the freed ring");

// out[t][j] = sum_{i < L} P[t][i] Q(j, i) in fp32 for the T x r pairs, one
// wave per pair: lane l sums (fused multiply-adds) elements 8 l + 512 m + e,
// m and e ascending, then a 64-lane xor tree; every lane ends with the same
// bits. Q(j, i) = Q[j][i] (QROW: A [r][K]) or Q[i][j] (B [N][r]).
// One wave computes pair w (whole waves; w >= T * r does nothing).
template <bool QROW>
__device__ __forceinline__ void rowdot_wave(const uint16_t* __restrict__ P,
                                            const uint16_t* __restrict__ Q, int T, int L, int r,
                                            float* __restrict__ out, int w) {
  if (w >= T * r) return;  // whole waves
  const int t = w / r, j = w - t * r;
  const int lane = threadIdx.x & 63;
  const uint16_t* prow = P + (int64_t)t * L;
  float acc = 0.f;
  for (int i0 = 8 * lane; i0 < L; i0 += 512) {
    const u32x4 pv = *reinterpret_cast<const u32x4*>(prow + i0);
    float pf[8], qf[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      pf[2 * e] = bf16_to_f32(pv[e] & 0xffffu);
      pf[2 * e + 1] = bf16_to_f32(pv[e] >> 16);
    }
    if constexpr (QROW) {
      const u32x4 qv = *reinterpret_cast<const u32x4*>(Q + (int64_t)j * L + i0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qf[2 * e] = bf16_to_f32(qv[e] & 0xffffu);
        qf[2 * e + 1] = bf16_to_f32(qv[e] >> 16);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[e] = bf16_to_f32(Q[(int64_t)(i0 + e) * r + j]);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf(pf[e], qf[e], acc);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc = acc + __shfl_xor(acc, off);
  if (lane == 0) out[w] = acc;
}

// A rank-r code job: out[t][j] = sum_i P[t][i] Q(j, i) for the T x r pairs,
// by `wgs` workgroups of four waves (0: none).
struct RowdotJob {
  const uint16_t* P;
  const uint16_t* Q;
  int L;
  float* out;
  int wgs;
};
inline int rowdot_wgs(int64_t T, int64_t r) { return (int)((T * r + 3) / 4); }

// Epilogue of a 64 x BN tile: out = bf16(acc + s * sum_j c[row][j] f[j][col]),
// c = the rows' rank-r codes (fp32 [T][r]), f = the adapter factor's columns
// (bf16, element (j, col) at F[col * fcs + j * fjs]). The ring is free on entry.
template <int BN, class Gm>
__device__ __forceinline__ void lora_epilogue(const Gm& gm, unsigned char* lds,
                                              const float* __restrict__ code,
                                              const uint16_t* __restrict__ F, int64_t fcs,
                                              int64_t fjs, int T, int ncols, int r, float scale,
                                              int row0, int col0, uint16_t* __restrict__ out,
                                              int64_t ldo) {
  float* cs = reinterpret_cast<float*>(lds);  // [r][64]
  float* fs = cs + kLoraBM * r;               // [r][BN]
  for (int i = threadIdx.x; i < kLoraBM * r; i += kThreads) {
    const int j = i / kLoraBM, rr = i - j * kLoraBM;
    cs[i] = row0 + rr < T ? code[(int64_t)(row0 + rr) * r + j] : 0.f;
  }
  for (int i = threadIdx.x; i < BN * r; i += kThreads) {
    const int j = i / BN, c = i - j * BN;
    fs[i] = col0 + c < ncols ? bf16_to_f32(F[(int64_t)(col0 + c) * fcs + (int64_t)j * fjs]) : 0.f;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int wm = wave % 2, wn = wave / 2;
#pragma unroll
  for (int i = 0; i < Gm::MI; ++i)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int row = wm * Gm::WTM + 16 * i + 4 * (lane >> 4) + rr;
#pragma unroll
      for (int jn = 0; jn < Gm::NJ; ++jn) {
        const int col = wn * Gm::WTN + 16 * jn + (lane & 15);
        float term = 0.f;
        for (int j = 0; j < r; ++j) term = fmaf(cs[j * kLoraBM + row], fs[j * BN + col], term);
        const float o = gm.acc[i][jn][rr] + scale * term;
        if (row0 + row < T && col0 + col < ncols)
          out[(int64_t)(row0 + row) * ldo + col0 + col] = (uint16_t)f32_to_bf16_rne(o);
      }
    }
}

// y tile of the forward (defined in rlk_lora_fwd.hip, instantiated for BN =
// 32, 64 and 128).
template <int BN>
__global__ void lora_fwd_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ W,
                                const float* __restrict__ u, const uint16_t* __restrict__ B, int T,
                                int K, int N, int r, float scale, int n_ttiles, int n_ntiles, int S,
                                uint16_t* __restrict__ y, float* __restrict__ part, RowdotJob ju);

}  // namespace rlk
