// rlk_microbench.hip — measured denominators for the roofline figures: a
// streaming copy and a streaming read (HBM bandwidth) and back-to-back
// independent bf16 MFMAs (matrix-core rate), declared in rlk_microbench.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rlk_device.h"
#include "rlk_internal.h"
#include "../../include/rlk_microbench.h"

namespace rlk {
namespace {

// 4 float4 per thread, strided by the grid so every load instruction of a
// wave covers 1 KB of consecutive bytes.
__global__ __launch_bounds__(kThreads) void copy_kernel(u32x4* __restrict__ dst,
                                                        const u32x4* __restrict__ src, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  const int64_t i0 = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  u32x4 v[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int64_t i = i0 + k * stride;
    if (i < n16) v[k] = src[i];
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int64_t i = i0 + k * stride;
    if (i < n16) dst[i] = v[k];
  }
}

// Linear read of `n_stages` 8 KB stages through LDS-DMA: workgroup b streams
// 1 MB runs (128 stages) b, b + grid, ... as one pipeline over a ring of 8
// slots, each wave moving two 1 KB blocks per stage. Nothing but the loads:
// the read rate HBM gives a consumer of contiguous bytes.
constexpr int kReadStages = 8;
__global__ __launch_bounds__(kThreads) void read_kernel(const unsigned char* __restrict__ src,
                                                        int64_t n_stages, float* __restrict__ sink) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[kReadStages * 8192];
  const int lane = threadIdx.x & 63, wave = wave_id();
  const uint32_t lds0 = lds_addr(lds);
  const int64_t runs = (n_stages + 127) / 128;
  const int64_t my_runs = (int64_t)blockIdx.x < runs ? (runs - 1 - blockIdx.x) / gridDim.x + 1 : 0;
  // stage j of this workgroup: run blockIdx.x + (j / 128) gridDim.x, stage j % 128 of it
  int64_t Q = 0;
  if (my_runs > 0) {
    const int64_t last_run = blockIdx.x + (my_runs - 1) * (int64_t)gridDim.x;
    const int64_t last_len = n_stages - 128 * last_run < 128 ? n_stages - 128 * last_run : 128;
    Q = (my_runs - 1) * 128 + last_len;
  }
  auto issue = [&](int64_t j) {
    const int64_t stage = 128 * ((int64_t)blockIdx.x + (j >> 7) * gridDim.x) + (j & 127);
    const i32x4 rs = make_rsrc(src + stage * 8192, 8192u);
    const uint32_t st = lds0 + (uint32_t)((j % kReadStages) * 8192);
    dma16(rs, st + 1024u * wave, 1024 * wave + 16 * lane, 0);
    dma16(rs, st + 1024u * (wave + 4), 1024 * (wave + 4) + 16 * lane, 0);
  };
  for (int64_t j = 0; j < kReadStages - 1 && j < Q; ++j) issue(j);
  for (int64_t j = 0; j < Q; ++j) {
    if (j + kReadStages - 2 < Q)
      wait_vmcnt<2 * (kReadStages - 2)>();
    else
      wait_vmcnt<0>();
    barrier_only();
    if (j + kReadStages - 1 < Q) issue(j + kReadStages - 1);
  }
  wait_vmcnt<0>();
  __syncthreads();
  const float v = reinterpret_cast<const float*>(lds)[threadIdx.x];
  if (v == -1.2345e-30f) sink[threadIdx.x & 3] = v;
}

// Every wave: 32 independent accumulators, `iters` rounds of one MFMA each;
// operands vary per lane so the data is not trivially constant.
__global__ __launch_bounds__(kThreads) void mfma_kernel(float* __restrict__ sink, int iters) {
  const int lane = threadIdx.x & 63;
  u32x4 ra, rb;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    ra[e] = 0x3c003c00u ^ (uint32_t)((lane * 2654435761u + e) & 0x007f007fu);
    rb[e] = 0x3c803c80u ^ (uint32_t)((lane * 40503u + 3 * e) & 0x007f007fu);
  }
  const bf16x8 a = __builtin_bit_cast(bf16x8, ra), b = __builtin_bit_cast(bf16x8, rb);
  f32x4 acc[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 32; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 32; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  // a value the compiler cannot predict decides the store
  if (s == -1.2345e-30f) sink[threadIdx.x & 3] = s;
}

typedef __attribute__((ext_vector_type(16))) float f32x16;

// The same back-to-back independent MFMAs in either instruction shape, with
// the shader clock (clock64: s_memtime) and the constant-rate wall clock
// (wall_clock64: s_memrealtime) read by lane 0 of wave 0 of every workgroup
// before and after; their ratio is the effective shader clock of the run.
// SHAPE 0: v_mfma_f32_16x16x32_bf16, 32 accumulators of 4 floats
// (32 x 16384 flops a round);
// SHAPE 1: v_mfma_f32_32x32x16_bf16, 16 accumulators of 16 floats
// (16 x 32768 flops a round: the same flops).
template <int SHAPE>
__global__ __launch_bounds__(kThreads) void mfma_clock_kernel(float* __restrict__ sink, int iters,
                                                              unsigned long long* __restrict__ clk) {
  const int lane = threadIdx.x & 63;
  u32x4 ra, rb;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    ra[e] = 0x3c003c00u ^ (uint32_t)((lane * 2654435761u + e) & 0x007f007fu);
    rb[e] = 0x3c803c80u ^ (uint32_t)((lane * 40503u + 3 * e) & 0x007f007fu);
  }
  const bf16x8 a = __builtin_bit_cast(bf16x8, ra), b = __builtin_bit_cast(bf16x8, rb);
  const bool timer = threadIdx.x == 0;
  unsigned long long c0 = 0, w0 = 0;
  if (timer) {
    c0 = clock64();
    w0 = wall_clock64();
  }
  float s = 0.f;
  if constexpr (SHAPE == 0) {
    f32x4 acc[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < 32; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 32; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  } else {
    f32x16 acc[16];
#pragma unroll
    for (int j = 0; j < 16; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < 16; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 16; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) s += acc[j][e];
  }
  if (timer) {
    // the accumulators feed s, so the reads below come after the MFMAs
    asm volatile("" ::"v"(s));
    const unsigned long long c1 = clock64(), w1 = wall_clock64();
    clk[2 * blockIdx.x] = c1 - c0;
    clk[2 * blockIdx.x + 1] = w1 - w0;
  }
  if (s == -1.2345e-30f) sink[threadIdx.x & 3] = s;
}

}  // namespace
}  // namespace rlk

extern "C" {

RLK_API rlk_status rlk_microbench_mfma_clock(float* sink, int64_t workgroups, int64_t iters,
                                             int shape, unsigned long long* clocks,
                                             int64_t* wall_clock_khz, void* stream) {
  if (!sink || (reinterpret_cast<uintptr_t>(sink) % 16) || !clocks ||
      (reinterpret_cast<uintptr_t>(clocks) % 16) || !wall_clock_khz || workgroups < 1 ||
      workgroups > (1 << 20) || iters < 1 || iters > (1 << 24) || (shape != 0 && shape != 1))
    return RLK_ERR_INVALID_ARG;
  const int s = rlk::check_device_status();
  if (s != RLK_OK) return (rlk_status)s;
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess)
    return RLK_ERR_HIP;
  *wall_clock_khz = khz;
  if (shape == 0)
    hipLaunchKernelGGL(rlk::mfma_clock_kernel<0>, dim3((unsigned)workgroups), dim3(rlk::kThreads), 0,
                       static_cast<hipStream_t>(stream), sink, (int)iters, clocks);
  else
    hipLaunchKernelGGL(rlk::mfma_clock_kernel<1>, dim3((unsigned)workgroups), dim3(rlk::kThreads), 0,
                       static_cast<hipStream_t>(stream), sink, (int)iters, clocks);
  return hipGetLastError() == hipSuccess ? RLK_OK : RLK_ERR_HIP;
}

RLK_API rlk_status rlk_microbench_copy(void* dst, const void* src, size_t bytes, void* stream) {
  if (!dst || !src || bytes == 0 || (bytes % 16) != 0 || bytes > (size_t(1) << 40))
    return RLK_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(dst) | reinterpret_cast<uintptr_t>(src)) % 16) return RLK_ERR_INVALID_ARG;
  const int s = rlk::check_device_status();
  if (s != RLK_OK) return (rlk_status)s;
  const int64_t n16 = (int64_t)(bytes / 16);
  const int64_t per_block = (int64_t)rlk::kThreads * 4;
  const int64_t grid = (n16 + per_block - 1) / per_block;
  hipLaunchKernelGGL(rlk::copy_kernel, dim3((unsigned)grid), dim3(rlk::kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<rlk::u32x4*>(dst),
                     static_cast<const rlk::u32x4*>(src), n16);
  return hipGetLastError() == hipSuccess ? RLK_OK : RLK_ERR_HIP;
}

RLK_API rlk_status rlk_microbench_read(const void* src, size_t bytes, float* sink, int64_t workgroups,
                                       void* stream) {
  if (!src || !sink || bytes == 0 || (bytes % 8192) != 0 || bytes > (size_t(1) << 40) ||
      workgroups < 1 || workgroups > (1 << 20))
    return RLK_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(sink)) % 16) return RLK_ERR_INVALID_ARG;
  const int s = rlk::check_device_status();
  if (s != RLK_OK) return (rlk_status)s;
  hipLaunchKernelGGL(rlk::read_kernel, dim3((unsigned)workgroups), dim3(rlk::kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const unsigned char*>(src),
                     (int64_t)(bytes / 8192), sink);
  return hipGetLastError() == hipSuccess ? RLK_OK : RLK_ERR_HIP;
}

RLK_API rlk_status rlk_microbench_mfma(float* sink, int64_t workgroups, int64_t iters, void* stream) {
  if (!sink || (reinterpret_cast<uintptr_t>(sink) % 16) || workgroups < 1 || workgroups > (1 << 20) ||
      iters < 1 || iters > (1 << 24))
    return RLK_ERR_INVALID_ARG;
  const int s = rlk::check_device_status();
  if (s != RLK_OK) return (rlk_status)s;
  hipLaunchKernelGGL(rlk::mfma_kernel, dim3((unsigned)workgroups), dim3(rlk::kThreads), 0,
                     static_cast<hipStream_t>(stream), sink, (int)iters);
  return hipGetLastError() == hipSuccess ? RLK_OK : RLK_ERR_HIP;
}

}  // extern "C"
