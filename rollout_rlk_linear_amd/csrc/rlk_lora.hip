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

#include "rlk_device.h"
#include "rlk_internal.h"
#include "rlk_lora_common.h"
#include "../../include/rlk_lora.h"

namespace rlk {
namespace {

// Splits of the forward's contraction over K: fixed by K alone (never by T,
// so every row's arithmetic is the same whatever the batch), about one per
// 1280 features, at most 4, each a multiple of 64.
inline int lora_ksplit(int64_t K) {
  for (int S = 4; S > 1; S /= 2)
    if (K >= 1280 * S && K % (64 * S) == 0) return S;
  return 1;
}

// The codes v = dy B (job jv, Q = B [N][r]) and u = x A^T (job ju, Q = A
// [r][K]) in one launch: workgroups 0 .. jv.wgs - 1 take jv, the rest ju. A
// split product launch runs the same jobs in extra workgroups of its own
// instead (its tiles do not read the codes; only its reduce does).
__global__ __launch_bounds__(kThreads) void lora_codes_kernel(int T, int r, RowdotJob jv,
                                                              RowdotJob ju) {
  const int b = (int)blockIdx.x;
  if (b < jv.wgs)
    rowdot_wave<false>(jv.P, jv.Q, T, jv.L, r, jv.out, b * (kThreads / 64) + wave_id());
  else
    rowdot_wave<true>(ju.P, ju.Q, T, ju.L, r, ju.out, (b - jv.wgs) * (kThreads / 64) + wave_id());
}

// y = bf16((part_0 + part_1 + ...) + s sum_j u[t][j] B[n][j]): workgroup b
// covers outputs 256 (b % nb) .. of row b / nb (nb = ceil(N / 256)), one a
// thread, the adapter term as the epilogue's fused multiply-add chain.
__global__ __launch_bounds__(kThreads) void lora_fwd_reduce_kernel(
    const float* __restrict__ part, const float* __restrict__ u, const uint16_t* __restrict__ B,
    int T, int N, int r, int S, float scale, uint16_t* __restrict__ y) {
  const int nb = (N + kThreads - 1) / kThreads;
  const int t = (int)blockIdx.x / nb;
  const int n = ((int)blockIdx.x - t * nb) * kThreads + (int)threadIdx.x;
  if (n >= N) return;
  const int64_t n_el = (int64_t)T * N;
  const int64_t i = (int64_t)t * N + n;
  float acc = part[i];
  for (int ks = 1; ks < S; ++ks) acc = acc + part[(int64_t)ks * n_el + i];
  const float* ut = u + (int64_t)t * r;
  const uint16_t* Bn = B + (int64_t)n * r;
  // the same ascending chain, its operands loaded ahead of it: B's row in
  // 16-byte pieces when r is a multiple of 8 (the row then starts 16-byte
  // aligned), else four elements at a time
  float term = 0.f;
  int j = 0;
  if ((r & 7) == 0) {
    for (; j < r; j += 8) {
      const u32x4 bv = *reinterpret_cast<const u32x4*>(Bn + j);
      float bb[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        bb[2 * e] = bf16_to_f32(bv[e] & 0xffffu);
        bb[2 * e + 1] = bf16_to_f32(bv[e] >> 16);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) term = fmaf(ut[j + e], bb[e], term);
    }
  }
  for (; j + 4 <= r; j += 4) {
    float uu[4], bb[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uu[e] = ut[j + e];
      bb[e] = bf16_to_f32(Bn[j + e]);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) term = fmaf(uu[e], bb[e], term);
  }
  for (; j < r; ++j) term = fmaf(ut[j], bf16_to_f32(Bn[j]), term);
  y[i] = (uint16_t)f32_to_bf16_rne(acc + scale * term);
}

// dx tile (64 tokens x 128 input features): dy W on the transposing mainloop,
// then + s v A with v = dy B. A's column k holds A[0..r-1][k]. With S > 1
// splits of the contraction over N (fixed by N alone) the tile covers split
// ns and writes its fp32 partial to part[ns][t][k]; lora_dx_reduce_kernel
// finishes dx.
// Workgroups past the tiles run the job jv (the codes v = dy B), then ju
// (u = x A^T), with S > 1 only.
__global__ __launch_bounds__(kThreads) void lora_dx_kernel(
    const uint16_t* __restrict__ dy, const uint16_t* __restrict__ W, const float* __restrict__ v,
    const uint16_t* __restrict__ A, int T, int K, int N, int r, float scale, int n_ttiles,
    int n_ktiles, int S, uint16_t* __restrict__ dx, float* __restrict__ part, RowdotJob jv,
    RowdotJob ju) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[LoraDxGemm::LDS_BYTES];
  const int n_main = n_ttiles * n_ktiles * S;
  if ((int)blockIdx.x >= n_main) {
    const int b = (int)blockIdx.x - n_main;
    if (b < jv.wgs)
      rowdot_wave<false>(jv.P, jv.Q, T, jv.L, r, jv.out, b * (kThreads / 64) + wave_id());
    else
      rowdot_wave<true>(ju.P, ju.Q, T, ju.L, r, ju.out,
                        (b - jv.wgs) * (kThreads / 64) + wave_id());
    return;
  }
  const int tt = (int)blockIdx.x % n_ttiles, rest = (int)blockIdx.x / n_ttiles;
  const int kt = rest % n_ktiles, ns = rest / n_ktiles;
  const int row0 = tt * kLoraBM, c0 = kt * kLoraBN;
  const int Ns = N / S;
  LoraDxGemm gm;
  gm.zero();
  gm.run(lds, dy + (int64_t)row0 * N, N, T - row0, W + c0, K, N, min(kLoraBN, K - c0), ns * Ns,
         (ns + 1) * Ns);
  if (S == 1) {
    lora_epilogue<kLoraBN>(gm, lds, v, A, 1, K, T, K, r, scale, row0, c0, dx, K);
    return;
  }
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int wm = wave % 2, wn = wave / 2;
  float* out = part + (int64_t)ns * T * K;
#pragma unroll
  for (int i = 0; i < LoraDxGemm::MI; ++i)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int row = row0 + wm * LoraDxGemm::WTM + 16 * i + 4 * (lane >> 4) + rr;
#pragma unroll
      for (int jn = 0; jn < LoraDxGemm::NJ; ++jn) {
        const int col = c0 + wn * LoraDxGemm::WTN + 16 * jn + (lane & 15);
        if (row < T && col < K) out[(int64_t)row * K + col] = gm.acc[i][jn][rr];
      }
    }
}

// dx = bf16((part_0 + part_1 + ...) + s sum_j v[t][j] A[j][k]), as
// lora_fwd_reduce_kernel with the code v and the factor A (column k holds
// A[0..r-1][k] at stride K).
__global__ __launch_bounds__(kThreads) void lora_dx_reduce_kernel(
    const float* __restrict__ part, const float* __restrict__ v, const uint16_t* __restrict__ A,
    int T, int K, int r, int S, float scale, uint16_t* __restrict__ dx) {
  const int nb = (K + kThreads - 1) / kThreads;
  const int t = (int)blockIdx.x / nb;
  const int k = ((int)blockIdx.x - t * nb) * kThreads + (int)threadIdx.x;
  if (k >= K) return;
  const int64_t n_el = (int64_t)T * K;
  const int64_t i = (int64_t)t * K + k;
  float acc = part[i];
  for (int ks = 1; ks < S; ++ks) acc = acc + part[(int64_t)ks * n_el + i];
  const float* vt = v + (int64_t)t * r;
  float term = 0.f;
  int j = 0;
  for (; j + 4 <= r; j += 4) {
    float vv[4], aa[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      vv[e] = vt[j + e];
      aa[e] = bf16_to_f32(A[(int64_t)(j + e) * K + k]);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) term = fmaf(vv[e], aa[e], term);
  }
  for (; j < r; ++j) term = fmaf(vt[j], bf16_to_f32(A[(int64_t)j * K + k]), term);
  dx[i] = (uint16_t)f32_to_bf16_rne(acc + scale * term);
}

// dA[j][k] = s * (fused multiply-add chain over t ascending of v[t][j] x[t][k]),
// and dB[n][j] = s * (the same over dy[t][n] u[t][j]), in one launch: the
// first da_blocks workgroups take dA (workgroup b: column block b % kb of row
// j = b / kb, kb = ceil(K / 256)), the rest dB (one output a thread).
__global__ __launch_bounds__(kThreads) void lora_dadb_kernel(
    const float* __restrict__ v, const uint16_t* __restrict__ x, const uint16_t* __restrict__ dy,
    const float* __restrict__ u, int T, int K, int N, int r, float scale, int da_blocks,
    float* __restrict__ da, float* __restrict__ db) {
  const int b = (int)blockIdx.x;
  if (b < da_blocks) {
    const int kb = (K + kThreads - 1) / kThreads;
    const int j = b / kb;
    const int k = (b - j * kb) * kThreads + (int)threadIdx.x;
    if (k >= K) return;
    // the ascending chain, its operands loaded eight at a time ahead of it
    float acc = 0.f;
    int t = 0;
    for (; t + 8 <= T; t += 8) {
      float a[8], c[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        a[e] = v[(int64_t)(t + e) * r + j];
        c[e] = bf16_to_f32(x[(int64_t)(t + e) * K + k]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fmaf(a[e], c[e], acc);
    }
    for (; t < T; ++t) acc = fmaf(v[(int64_t)t * r + j], bf16_to_f32(x[(int64_t)t * K + k]), acc);
    da[(int64_t)j * K + k] = scale * acc;
    return;
  }
  const int64_t i = (int64_t)(b - da_blocks) * kThreads + threadIdx.x;
  if (i >= (int64_t)N * r) return;
  const int n = (int)(i / r), j = (int)(i - (int64_t)n * r);
  float acc = 0.f;
  int t = 0;
  for (; t + 8 <= T; t += 8) {
    float a[8], c[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] = bf16_to_f32(dy[(int64_t)(t + e) * N + n]);
      c[e] = u[(int64_t)(t + e) * r + j];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf(a[e], c[e], acc);
  }
  for (; t < T; ++t) acc = fmaf(bf16_to_f32(dy[(int64_t)t * N + n]), u[(int64_t)t * r + j], acc);
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

// u and v (fp32 [T][r] each), then the split partials: the forward's
// (fp32 [S][T][N], S = lora_ksplit(K)) or dx's (fp32 [S'][T][K], S' =
// lora_ksplit(N)), whichever is larger.
size_t lora_ws(int64_t T, int64_t K, int64_t N, int64_t r) {
  const int S = lora_ksplit(K), Sx = lora_ksplit(N);
  const size_t uv = (size_t(2) * T * r * 4 + 255) / 256 * 256;
  const size_t pf = S > 1 ? size_t(S) * T * N * 4 : 0;
  const size_t px = Sx > 1 ? size_t(Sx) * T * K * 4 : 0;
  return uv + ((pf > px ? pf : px) + 255) / 256 * 256;
}

}  // namespace
}  // namespace rlk

extern "C" {

RLK_API size_t rlk_lora_linear_workspace_bytes(int64_t T, int64_t K, int64_t N, int64_t r) {
  if (T <= 0 || rlk::lora_shape(T, K, N, r) != RLK_OK) return 0;
  return rlk::lora_ws(T, K, N, r);
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
  if (workspace_bytes < rlk::lora_ws(T, K, N, r)) return RLK_ERR_WORKSPACE_TOO_SMALL;
  s = (rlk_status)rlk::check_device_status();
  if (s != RLK_OK) return s;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const auto* xb = static_cast<const uint16_t*>(x);
  const auto* Wb = static_cast<const uint16_t*>(weight);
  const auto* Ab = static_cast<const uint16_t*>(lora_a);
  const auto* Bb = static_cast<const uint16_t*>(lora_b);
  float* u = static_cast<float*>(workspace);
  float* part = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                         (size_t(2) * T * r * 4 + 255) / 256 * 256);
  const int nt = rlk::cdiv_i(T, rlk::kLoraBM);
  const int S = rlk::lora_ksplit(K);
  uint16_t* yb = static_cast<uint16_t*>(y);
  // u = x A^T: with S > 1 only the reduce reads it, so extra workgroups of
  // the product launch compute it; with S = 1 the tiles' epilogue needs it first
  rlk::RowdotJob ju{xb, Ab, (int)K, u, rlk::rowdot_wgs(T, r)};
  if (S == 1) {
    const rlk::RowdotJob none{nullptr, nullptr, 0, nullptr, 0};
    hipLaunchKernelGGL(rlk::lora_codes_kernel, dim3(ju.wgs), dim3(rlk::kThreads), 0, st, (int)T,
                       (int)r, none, ju);
    ju.wgs = 0;
  }
  // narrower tiles when the wide ones would leave most compute units idle
  // (the tile width does not change any element's arithmetic)
  if ((int64_t)nt * rlk::cdiv_i(N, rlk::kLoraBN) * S >= 256) {
    const int nn = rlk::cdiv_i(N, rlk::kLoraBN);
    hipLaunchKernelGGL(rlk::lora_fwd_kernel<rlk::kLoraBN>, dim3(nt * nn * S + ju.wgs),
                       dim3(rlk::kThreads), 0, st, xb, Wb, u, Bb, (int)T, (int)K, (int)N, (int)r,
                       scale, nt, nn, S, yb, part, ju);
  } else if ((int64_t)nt * rlk::cdiv_i(N, rlk::kLoraBNm) * S >= 256) {
    const int nn = rlk::cdiv_i(N, rlk::kLoraBNm);
    hipLaunchKernelGGL(rlk::lora_fwd_kernel<rlk::kLoraBNm>, dim3(nt * nn * S + ju.wgs),
                       dim3(rlk::kThreads), 0, st, xb, Wb, u, Bb, (int)T, (int)K, (int)N, (int)r,
                       scale, nt, nn, S, yb, part, ju);
  } else {
    const int nn = rlk::cdiv_i(N, rlk::kLoraBNs);
    hipLaunchKernelGGL(rlk::lora_fwd_kernel<rlk::kLoraBNs>, dim3(nt * nn * S + ju.wgs),
                       dim3(rlk::kThreads), 0, st, xb, Wb, u, Bb, (int)T, (int)K, (int)N, (int)r,
                       scale, nt, nn, S, yb, part, ju);
  }
  if (S > 1)
    hipLaunchKernelGGL(rlk::lora_fwd_reduce_kernel, dim3(T * rlk::cdiv_i(N, rlk::kThreads)),
                       dim3(rlk::kThreads), 0, st, part, u, Bb, (int)T, (int)N, (int)r, S, scale,
                       yb);
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
  if (workspace_bytes < rlk::lora_ws(T, K, N, r)) return RLK_ERR_WORKSPACE_TOO_SMALL;
  s = (rlk_status)rlk::check_device_status();
  if (s != RLK_OK) return s;
  const auto* xb = static_cast<const uint16_t*>(x);
  const auto* Wb = static_cast<const uint16_t*>(weight);
  const auto* Ab = static_cast<const uint16_t*>(lora_a);
  const auto* Bb = static_cast<const uint16_t*>(lora_b);
  const auto* dyb = static_cast<const uint16_t*>(dy);
  float* u = static_cast<float*>(workspace);
  float* v = u + T * r;
  // v = dy B (for dx and dA) and u = x A^T (for dB): with a split
  // contraction of dx (Sx > 1) its tiles do not read v, so extra workgroups
  // of the dx launch compute both; otherwise one launch of their own
  const int Sx = rlk::lora_ksplit(N);
  const bool fold = dx && Sx > 1;
  rlk::RowdotJob jv{dyb, Bb, (int)N, v, (dx || da) ? rlk::rowdot_wgs(T, r) : 0};
  rlk::RowdotJob ju{xb, Ab, (int)K, u, db ? rlk::rowdot_wgs(T, r) : 0};
  if (!fold) {
    if (jv.wgs + ju.wgs > 0)
      hipLaunchKernelGGL(rlk::lora_codes_kernel, dim3(jv.wgs + ju.wgs), dim3(rlk::kThreads), 0,
                         st, (int)T, (int)r, jv, ju);
    jv.wgs = ju.wgs = 0;
  }
  if (dx) {
    const int nt = rlk::cdiv_i(T, rlk::kLoraBM);
    const int nk = rlk::cdiv_i(K, rlk::kLoraBN);
    float* part = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                           (size_t(2) * T * r * 4 + 255) / 256 * 256);
    hipLaunchKernelGGL(rlk::lora_dx_kernel, dim3(nt * nk * Sx + jv.wgs + ju.wgs),
                       dim3(rlk::kThreads), 0, st, dyb, Wb, v, Ab, (int)T, (int)K, (int)N,
                       (int)r, scale, nt, nk, Sx, static_cast<uint16_t*>(dx), part, jv, ju);
    if (Sx > 1)
      hipLaunchKernelGGL(rlk::lora_dx_reduce_kernel, dim3(T * rlk::cdiv_i(K, rlk::kThreads)),
                         dim3(rlk::kThreads), 0, st, part, v, Ab, (int)T, (int)K, (int)r, Sx, scale,
                         static_cast<uint16_t*>(dx));
  }
  const int da_blocks = da ? rlk::cdiv_i(K, rlk::kThreads) * (int)r : 0;
  const int db_blocks = db ? rlk::cdiv_i(N * r, rlk::kThreads) : 0;
  if (da_blocks + db_blocks > 0)
    hipLaunchKernelGGL(rlk::lora_dadb_kernel, dim3(da_blocks + db_blocks), dim3(rlk::kThreads), 0,
                       st, v, xb, dyb, u, (int)T, (int)K, (int)N, (int)r, scale, da_blocks, da,
                       db);
  return hipGetLastError() == hipSuccess ? RLK_OK : RLK_ERR_HIP;
}

}  // extern "C"
