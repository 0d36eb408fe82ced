/* rlk_lora.h — batch-invariant LoRA linear on gfx950 (MI355X).
 *
 * The layer of the runtime report's gate for low-rank adapters (page
 * "RL-Kernel h3-runtime-integration-b200 report.json", key lora_gate): a
 * linear layer whose base weight is frozen, with a trainable rank-r adapter.
 * The report checks, on shapes N512 K384 T70, N2048 K1024 T257 and
 * N5120 K5120 T33, that it is repeatable, that forward rows are independent
 * and that the forward output and the gradients of x, A and B are close to
 * float64 in the norm-wise relative error. The layer (the plain reading of an
 * adapter on a frozen linear) is, for each token row x_t:
 *
 *   y_t = W x_t + s * B (A x_t)
 *
 * with W bf16 [N,K] (frozen), A bf16 [r,K], B bf16 [N,r], a scalar scale s,
 * x bf16 [T,K] and y bf16 [T,N]. With u = x A^T and the output gradient dy:
 *
 *   dx = dy W + s (dy B) A,   dA = s (dy B)^T x,   dB = s dy^T u
 *
 * and no gradient for W.
 *
 * Numerics (fixed, whatever T and the row's position in the batch):
 *   - x W^T and dy W: bf16 MFMA chains over K (resp. N) ascending in steps of
 *     32 from zero, fp32 accumulation. A long contraction is cut into S
 *     equal splits, S fixed by its length L alone (the largest of 4, 2 with
 *     L >= 1280 S and L a multiple of 64 S, else 1): each split is such a
 *     chain over its own range, and the split sums are added in ascending
 *     split order (((p0 + p1) + p2) + p3) before the adapter term;
 *   - u[t][j] = sum_k x[t][k] A[j][k] and v[t][j] = sum_n dy[t][n] B[n][j] in
 *     fp32: lane l of a wave sums, with fused multiply-adds, the elements
 *     8 l + 512 m + e (m ascending, e = 0..7 ascending), then a 64-lane xor
 *     tree (offsets 32, 16, ..., 1);
 *   - the adapter term of an output element is the fused multiply-add chain
 *     over j = 0 .. r-1 of u (or v) with B (or A), then out = acc + s * term,
 *     rounded to bf16 (nearest even);
 *   - dA[j][k] = s * (fused multiply-add chain over t = 0 .. T-1 of
 *     v[t][j] x[t][k]) and dB[n][j] = s * (the same chain of dy[t][n] u[t][j]),
 *     fp32. These two are sums over rows: repeatable bit for bit, not
 *     independent of the batch.
 * So every row of y and of dx is bitwise independent of the other rows.
 *
 * Conventions as in rlk_linear.h: device pointers owned by the caller,
 * 16-byte aligned; all work enqueued on `stream`; the library allocates
 * nothing (the caller's workspace); every argument error is returned before
 * any launch; no fallback path.
 * Limits: K and N multiples of 64, K <= 65536, N <= 2^20, 1 <= r <= 64,
 * T <= 2^21 (RLK_ERR_UNSUPPORTED_SHAPE otherwise).
 */
#ifndef RLK_LORA_H
#define RLK_LORA_H

#include "rlk_linear.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes of device workspace for a forward or backward call: u and v, fp32
 * [T][r] each, rounded up to 256 bytes. 0 when T == 0 or a size is invalid. */
RLK_API size_t rlk_lora_linear_workspace_bytes(int64_t T, int64_t K, int64_t N, int64_t r);

/* Forward: y = x W^T + scale * (x A^T) B^T, y bf16 [T,N] (overwritten).
 * T == 0 is a no-op. */
RLK_API rlk_status rlk_lora_linear_fwd(const void* x, const void* weight, const void* lora_a,
                                       const void* lora_b, int64_t T, int64_t K, int64_t N,
                                       int64_t r, float scale, void* y, void* workspace,
                                       size_t workspace_bytes, void* stream);

/* Backward from dy bf16 [T,N]: dx bf16 [T,K], dA fp32 [r,K], dB fp32 [N,r],
 * each overwritten, each optional (NULL = skip; at least one). T == 0 writes
 * zeros to dA and dB. */
RLK_API rlk_status rlk_lora_linear_bwd(const void* x, const void* weight, const void* lora_a,
                                       const void* lora_b, const void* dy, int64_t T, int64_t K,
                                       int64_t N, int64_t r, float scale, void* dx, float* da,
                                       float* db, void* workspace, size_t workspace_bytes,
                                       void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RLK_LORA_H */
