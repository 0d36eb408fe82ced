/* rlk_microbench.h — on-device microbenchmarks that give the measured
 * denominators of the roofline figures: sustained HBM copy and read bandwidth and the
 * sustained dense bf16 MFMA rate of the same v_mfma_f32_16x16x32_bf16
 * instruction the GEMM kernels use. They are measurement tools, not part of
 * the linear log-prob path.
 *
 * Both calls only enqueue work on `stream` (a hipStream_t; NULL = the null
 * stream) and return immediately; the caller times them with events on that
 * stream. They allocate nothing. Errors: RLK_ERR_INVALID_ARG for NULL or
 * misaligned pointers or sizes out of range, RLK_ERR_UNSUPPORTED_DEVICE when
 * the current device is not gfx950, RLK_ERR_HIP when the launch fails.
 */
#ifndef RLK_MICROBENCH_H
#define RLK_MICROBENCH_H

#include "rlk_linear.h"

#ifdef __cplusplus
extern "C" {
#endif

/* dst[i] = src[i] for `bytes` bytes (a multiple of 16, at most 2^40), both
 * device pointers 16-byte aligned, not overlapping. One read and one write
 * of every byte: count 2 * bytes of HBM traffic. */
RLK_API rlk_status rlk_microbench_copy(void* dst, const void* src, size_t bytes, void* stream);

/* Reads `bytes` bytes of src (device, 16-byte aligned; a multiple of 8192, at
 * most 2^40) once, linearly, into LDS through LDS-DMA and discards them:
 * `workgroups` workgroups (1 .. 2^20; one per compute unit is the intended
 * use) each stream 1 MB runs over a ring of eight 8 KB stages. Counts
 * `bytes` of HBM traffic. sink as for rlk_microbench_mfma. */
RLK_API rlk_status rlk_microbench_read(const void* src, size_t bytes, float* sink, int64_t workgroups,
                                       void* stream);

/* Back-to-back independent bf16 MFMAs (16x16x32, fp32 accumulate) on every
 * SIMD: `workgroups` workgroups of 4 waves, each wave `iters` rounds of 32
 * MFMAs (1 <= iters <= 2^24, 1 <= workgroups <= 2^20). Flops performed:
 * workgroups * 4 * iters * 32 * 16384. `sink` (device, 16-byte aligned,
 * >= 16 bytes) receives a value derived from the accumulators so the work
 * cannot be elided. */
RLK_API rlk_status rlk_microbench_mfma(float* sink, int64_t workgroups, int64_t iters, void* stream);

/* The MFMA rate in either instruction shape, with the clock it ran at:
 * shape 0 = v_mfma_f32_16x16x32_bf16 (32 independent accumulators per wave),
 * shape 1 = v_mfma_f32_32x32x16_bf16 (16 accumulators of 16 floats); both do
 * the flops of rlk_microbench_mfma for the same workgroups and iters. Lane 0 of
 * wave 0 of every workgroup writes clocks[2 b] = shader-clock cycles
 * (clock64) and clocks[2 b + 1] = wall-clock ticks (wall_clock64) between
 * its start and its end; *wall_clock_khz (host) receives the wall clock's
 * rate, so sum(clocks[2 b]) / sum(clocks[2 b + 1]) * rate is the effective
 * shader clock. clocks: device, 16-byte aligned, 2 * workgroups entries. */
RLK_API rlk_status rlk_microbench_mfma_clock(float* sink, int64_t workgroups, int64_t iters,
                                             int shape, unsigned long long* clocks,
                                             int64_t* wall_clock_khz, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RLK_MICROBENCH_H */
