// rlk_lora.hip — batch-invariant LoRA linear for gfx950: y = x W^T + s (x A^T) B^T
// and its gradients dx, dA, dB (W frozen), declared in include/rlk_lora.h.
//
// The base products are the library's LDS-DMA MFMA mainloops: x W^T is a
// K-contiguous x K-contiguous product (AsyncGemmP, as the logits), dy W is a
// K-contiguous x K-major product (AsyncGemmKN, as dH). The rank-r adapter
// enters in the epilogue of each tile in fp32. Every output element of y and
// dx is computed by the same instruction sequence whatever T, the tile shape
// or the row's position, so rows are bitwise independent of the batch.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rlk_device.cuh"
#include "rlk_internal.h"
#include "../../include/rlk_lora.h"

namespace rlk {
namespace {

constexpr int kLoraBM = 64;    // rows (tokens) per tile
constexpr int kLoraBN = 128;   // output columns per tile
constexpr int kLoraMaxRank = 64;
using LoraFwdGemm = AsyncGemmP<kLoraBM, kLoraBN, 2, 2>;
using LoraDxGemm = AsyncGemmKN<kLoraBM, kLoraBN, 2, 2, 4>;
static_assert((kLoraBM + kLoraBN) * kLoraMaxRank * 4 <= LoraFwdGemm::LDS_BYTES &&
                  (kLoraBM + kLoraBN) * kLoraMaxRank * 4 <= LoraDxGemm::LDS_BYTES,
              "the adapter operands of a tile fit the freed ring");

// out[t][j] = sum_{i < L} P[t][i] Q(j, i) in fp32 for the T x r pairs, one
// wave per pair: lane l sums (fused multiply-adds) elements 8 l + 512 m + e,
// m and e ascending, then a 64-lane xor tree; every lane ends with the same
// bits. Q(j, i) = Q[j][i] (QROW: A [r][K]) or Q[i][j] (B [N][r]).
template <bool QROW>
__global__ __launch_bounds__(kThreads) void lora_rowdot_kernel(const uint16_t* __restrict__ P,
                                                               const uint16_t* __restrict__ Q,
                                                               int T, int L, int r,
                                                               float* __restrict__ out) {
  const int w = (int)blockIdx.x * (kThreads / 64) + wave_id();
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

// Epilogue of a 64 x 128 tile: out = bf16(acc + s * sum_j c[row][j] f[j][col]),
// c = the rows' rank-r codes (fp32 [T][r]), f = the adapter factor's columns
// (bf16, element (j, col) at F[col * fcs + j * fjs]). The ring is free on entry.
template <class Gm>
__device__ __forceinline__ void lora_epilogue(const Gm& gm, unsigned char* lds,
                                              const float* __restrict__ code,
                                              const uint16_t* __restrict__ F, int64_t fcs,
                                              int64_t fjs, int T, int ncols, int r, float scale,
                                              int row0, int col0, uint16_t* __restrict__ out,
                                              int64_t ldo) {
  float* cs = reinterpret_cast<float*>(lds);  // [r][64]
  float* fs = cs + kLoraBM * r;               // [r][128]
  for (int i = threadIdx.x; i < kLoraBM * r; i += kThreads) {
    const int j = i / kLoraBM, rr = i - j * kLoraBM;
    cs[i] = row0 + rr < T ? code[(int64_t)(row0 + rr) * r + j] : 0.f;
  }
  for (int i = threadIdx.x; i < kLoraBN * r; i += kThreads) {
    const int j = i / kLoraBN, c = i - j * kLoraBN;
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
        for (int j = 0; j < r; ++j) term = fmaf(cs[j * kLoraBM + row], fs[j * kLoraBN + col], term);
        const float o = gm.acc[i][jn][rr] + scale * term;
        if (row0 + row < T && col0 + col < ncols)
          out[(int64_t)(row0 + row) * ldo + col0 + col] = (uint16_t)f32_to_bf16_rne(o);
      }
    }
}

// y tile (64 tokens x 128 outputs): x W^T on the MFMA mainloop, then + s u B^T.
__global__ __launch_bounds__(kThreads) void lora_fwd_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ W, const float* __restrict__ u,
    const uint16_t* __restrict__ B, int T, int K, int N, int r, float scale, int n_ttiles,
    uint16_t* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[LoraFwdGemm::LDS_BYTES];
  const int tt = (int)blockIdx.x % n_ttiles, nt = (int)blockIdx.x / n_ttiles;
  const int row0 = tt * kLoraBM, col0 = nt * kLoraBN;
  LoraFwdGemm gm;
  gm.zero();
  gm.run(lds, x + (int64_t)row0 * K, K, T - row0, W + (int64_t)col0 * K, K, N - col0, 0, K);
  // run() ends on a barrier: the ring is free. B's column n holds B[n][0..r-1].
  lora_epilogue(gm, lds, u, B, r, 1, T, N, r, scale, row0, col0, y, N);
}

// dx tile (64 tokens x 128 input features): dy W on the transposing mainloop,
// then + s v A with v = dy B. A's column k holds A[0..r-1][k].
__global__ __launch_bounds__(kThreads) void lora_dx_kernel(
    const uint16_t* __restrict__ dy, const uint16_t* __restrict__ W, const float* __restrict__ v,
    const uint16_t* __restrict__ A, int T, int K, int N, int r, float scale, int n_ttiles,
    uint16_t* __restrict__ dx) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[LoraDxGemm::LDS_BYTES];
  const int tt = (int)blockIdx.x % n_ttiles, kt = (int)blockIdx.x / n_ttiles;
  const int row0 = tt * kLoraBM, c0 = kt * kLoraBN;
  LoraDxGemm gm;
  gm.zero();
  gm.run(lds, dy + (int64_t)row0 * N, N, T - row0, W + c0, K, N, min(kLoraBN, K - c0), 0, N);
  lora_epilogue(gm, lds, v, A, 1, K, T, K, r, scale, row0, c0, dx, K);
}

// dA[j][k] = s * (fused multiply-add chain over t ascending of v[t][j] x[t][k]).
__global__ __launch_bounds__(kThreads) void lora_da_kernel(const float* __restrict__ v,
                                                           const uint16_t* __restrict__ x, int T,
                                                           int K, int r, float scale,
                                                           float* __restrict__ da) {
  const int k = (int)blockIdx.x * kThreads + threadIdx.x;
  const int j = (int)blockIdx.y;
  if (k >= K) return;
  float acc = 0.f;
  for (int t = 0; t < T; ++t)
    acc = fmaf(v[(int64_t)t * r + j], bf16_to_f32(x[(int64_t)t * K + k]), acc);
  da[(int64_t)j * K + k] = scale * acc;
}

// dB[n][j] = s * (fused multiply-add chain over t ascending of dy[t][n] u[t][j]).
__global__ __launch_bounds__(kThreads) void lora_db_kernel(const uint16_t* __restrict__ dy,
                                                           const float* __restrict__ u, int T,
                                                           int N, int r, float scale,
                                                           float* __restrict__ db) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= (int64_t)N * r) return;
  const int n = (int)(i / r), j = (int)(i - (int64_t)n * r);
  float acc = 0.f;
  for (int t = 0; t < T; ++t)
    acc = fmaf(bf16_to_f32(dy[(int64_t)t * N + n]), u[(int64_t)t * r + j], acc);
  db[i] = scale * acc;
}

inline int cdiv_i(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

inline bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

rlk_status lora_shape(int64_t T, int64_t K, int64_t N, int64_t r) {
  if (T < 0 || K <= 0 || N <= 0 || r < 1) return RLK_ERR_INVALID_ARG;
  if (K % 64 || N % 64 || K > 65536 || N > (int64_t(1) << 20) || r > kLoraMaxRank ||
      T > (int64_t(1) << 21))
    return RLK_ERR_UNSUPPORTED_SHAPE;
  return RLK_OK;
}

size_t lora_ws(int64_t T, int64_t r) { return (size_t(2) * T * r * 4 + 255) / 256 * 256; }

}  // namespace
}  // namespace rlk

extern "C" {

RLK_API size_t rlk_lora_linear_workspace_bytes(int64_t T, int64_t K, int64_t N, int64_t r) {
  if (T <= 0 || rlk::lora_shape(T, K, N, r) != RLK_OK) return 0;
  return rlk::lora_ws(T, r);
}

RLK_API rlk_status rlk_lora_linear_fwd(const void* x, const void* weight, const void* lora_a,
                                       const void* lora_b, int64_t T, int64_t K, int64_t N,
                                       int64_t r, float scale, void* y, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  rlk_status s = rlk::lora_shape(T, K, N, r);
  if (s != RLK_OK) return s;
  if (T == 0) return RLK_OK;
  if (!x || !weight || !lora_a || !lora_b || !y || !workspace) return RLK_ERR_INVALID_ARG;
  if (!rlk::al16(x) || !rlk::al16(weight) || !rlk::al16(lora_a) || !rlk::al16(lora_b) ||
      !rlk::al16(y) || !rlk::al16(workspace))
    return RLK_ERR_INVALID_ARG;
  if (workspace_bytes < rlk::lora_ws(T, r)) return RLK_ERR_WORKSPACE_TOO_SMALL;
  s = (rlk_status)rlk::check_device_status();
  if (s != RLK_OK) return s;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const auto* xb = static_cast<const uint16_t*>(x);
  const auto* Wb = static_cast<const uint16_t*>(weight);
  const auto* Ab = static_cast<const uint16_t*>(lora_a);
  const auto* Bb = static_cast<const uint16_t*>(lora_b);
  float* u = static_cast<float*>(workspace);
  hipLaunchKernelGGL(rlk::lora_rowdot_kernel<true>, dim3(rlk::cdiv_i(T * r, 4)), dim3(rlk::kThreads),
                     0, st, xb, Ab, (int)T, (int)K, (int)r, u);
  const int nt = rlk::cdiv_i(T, rlk::kLoraBM);
  hipLaunchKernelGGL(rlk::lora_fwd_kernel, dim3(nt * rlk::cdiv_i(N, rlk::kLoraBN)),
                     dim3(rlk::kThreads), 0, st, xb, Wb, u, Bb, (int)T, (int)K, (int)N, (int)r,
                     scale, nt, static_cast<uint16_t*>(y));
  return hipGetLastError() == hipSuccess ? RLK_OK : RLK_ERR_HIP;
}

RLK_API rlk_status rlk_lora_linear_bwd(const void* x, const void* weight, const void* lora_a,
                                       const void* lora_b, const void* dy, int64_t T, int64_t K,
                                       int64_t N, int64_t r, float scale, void* dx, float* da,
                                       float* db, void* workspace, size_t workspace_bytes,
                                       void* stream) {
  rlk_status s = rlk::lora_shape(T, K, N, r);
  if (s != RLK_OK) return s;
  if (!dx && !da && !db) return RLK_ERR_INVALID_ARG;
  if ((dx && !rlk::al16(dx)) || (da && !rlk::al16(da)) || (db && !rlk::al16(db)))
    return RLK_ERR_INVALID_ARG;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (T == 0) {
    s = (rlk_status)rlk::check_device_status();
    if (s != RLK_OK) return s;
    if (da && rlk::launch_fill_zero(da, r * K, st) != hipSuccess) return RLK_ERR_HIP;
    if (db && rlk::launch_fill_zero(db, N * r, st) != hipSuccess) return RLK_ERR_HIP;
    return RLK_OK;
  }
  if (!x || !weight || !lora_a || !lora_b || !dy || !workspace) return RLK_ERR_INVALID_ARG;
  if (!rlk::al16(x) || !rlk::al16(weight) || !rlk::al16(lora_a) || !rlk::al16(lora_b) ||
      !rlk::al16(dy) || !rlk::al16(workspace))
    return RLK_ERR_INVALID_ARG;
  if (workspace_bytes < rlk::lora_ws(T, r)) return RLK_ERR_WORKSPACE_TOO_SMALL;
  s = (rlk_status)rlk::check_device_status();
  if (s != RLK_OK) return s;
  const auto* xb = static_cast<const uint16_t*>(x);
  const auto* Wb = static_cast<const uint16_t*>(weight);
  const auto* Ab = static_cast<const uint16_t*>(lora_a);
  const auto* Bb = static_cast<const uint16_t*>(lora_b);
  const auto* dyb = static_cast<const uint16_t*>(dy);
  float* u = static_cast<float*>(workspace);
  float* v = u + T * r;
  const dim3 pairs(rlk::cdiv_i(T * r, 4));
  if (dx || da)
    hipLaunchKernelGGL(rlk::lora_rowdot_kernel<false>, pairs, dim3(rlk::kThreads), 0, st, dyb, Bb,
                       (int)T, (int)N, (int)r, v);
  if (db)
    hipLaunchKernelGGL(rlk::lora_rowdot_kernel<true>, pairs, dim3(rlk::kThreads), 0, st, xb, Ab,
                       (int)T, (int)K, (int)r, u);
  if (dx) {
    const int nt = rlk::cdiv_i(T, rlk::kLoraBM);
    hipLaunchKernelGGL(rlk::lora_dx_kernel, dim3(nt * rlk::cdiv_i(K, rlk::kLoraBN)),
                       dim3(rlk::kThreads), 0, st, dyb, Wb, v, Ab, (int)T, (int)K, (int)N, (int)r,
                       scale, nt, static_cast<uint16_t*>(dx));
  }
  if (da)
    hipLaunchKernelGGL(rlk::lora_da_kernel, dim3(rlk::cdiv_i(K, rlk::kThreads), (unsigned)r),
                       dim3(rlk::kThreads), 0, st, v, xb, (int)T, (int)K, (int)r, scale, da);
  if (db)
    hipLaunchKernelGGL(rlk::lora_db_kernel, dim3(rlk::cdiv_i(N * r, rlk::kThreads)),
                       dim3(rlk::kThreads), 0, st, dyb, u, (int)T, (int)N, (int)r, scale, db);
  return hipGetLastError() == hipSuccess ? RLK_OK : RLK_ERR_HIP;
}

}  // extern "C"
