/*
 * rlk_linear.h — C ABI of the fused, batch-invariant linear log-prob for
 * MI355X (gfx950).
 *
 * The operator. Per token t, with hidden h_t (bf16, H values), the LM-head
 * weight W (bf16, V_total rows of H) and a target id y_t, the logits are
 * z_t = W h_t and the op returns
 *     logp_t    = z_{t,y_t} - log sum_v exp(z_{t,v})
 *     entropy_t = -sum_v p_{t,v} log p_{t,v},   p_t = softmax(z_t)   (nats)
 * and, in the backward pass, the gradients of sum_t (dlogp_t logp_t +
 * dentropy_t entropy_t) with respect to the hidden states and W. It is the
 * linear-logp provider that stands in for VIME's
 * calculate_log_probs_and_entropy (page "VIME Qwen3-8B TP4/CP2 200-round
 * consistency experiment", section "User-facing operator matrix"), whose
 * train-side and rollout-side log-probs must agree bit for bit (page
 * "RL-Kernel evidence h100-cp-gradient.json",
 * validation.train_rollout_logprob: require_exact, 0 bitwise mismatches).
 *
 * Bitwise contract. For a fixed build, every output row (logp, entropy,
 * stats, and each row of dhidden) depends only on that row's hidden vector,
 * its target, its upstream gradients and W: not on T, on the other rows, on
 * the row's position in the batch, or on the repeat. dweight is a sum over
 * rows and is only repeat-deterministic. Nothing uses atomics; every
 * reduction runs in a fixed order set by the vocabulary layout alone.
 *
 * Memory. All tensor pointers are device pointers owned by the caller,
 * row-major, 16-byte aligned; inputs and outputs must not alias. The library
 * allocates nothing: scratch memory is the caller's `workspace` (size from the
 * *_workspace_bytes queries). It keeps no pointer after a call returns.
 *
 * Streams. `stream` is a hipStream_t (NULL = the null stream). Calls enqueue
 * kernels and return without synchronising; device faults surface at the
 * caller's next synchronisation.
 *
 * Errors. Every argument error is reported before anything is launched, by a
 * status code (nothing is thrown across the ABI, nothing aborts). There is no
 * fallback path of any kind: the op either runs the gfx950 kernels or returns
 * an error.
 *
 * Vocabulary slices. A call may cover rows [vocab_start, vocab_start + V) of
 * a vocabulary of vocab_total rows (one GPU's share of a tensor-parallel LM
 * head; the pages' actor runs at TP=4). `weight` then points at the slice's
 * first row. The forward returns the slice's partial statistics, which
 * rlk_linear_logp_combine (on the device) or rlk_linear_logp_combine_host
 * merges across slices; the backward takes the merged (whole-vocabulary)
 * statistics.
 *
 * Tensor-parallel invariance. When vocab_total is a multiple of 4 the
 * vocabulary is cut into 4 virtual slices of vocab_total / 4 rows. The
 * forward reduces each virtual slice on its own (groups of 256 columns from
 * the slice's first row) and merges the virtual slices with a fixed balanced
 * tree, ((s0 + s1) + (s2 + s3)). A call that covers 1, 2 or all 4 virtual
 * slices, aligned to its own size (TP = 4, 2 or 1 with equal shares), computes
 * exactly its subtree, and rlk_linear_logp_combine merges call records with
 * the same tree: so TP = 1, 2 and 4 give identical bits for logp, entropy and
 * stats. The backward does the same for dhidden: each virtual slice's
 * contribution sum_{v in slice} G[t,v] W[v,:] is summed over splits that start
 * at the slice's first row and are sized by the slice alone, and the slices'
 * fp32 contributions are added by the same tree before the bf16 rounding; a
 * slice call returns its subtree in fp32 (RLK_DH_F32) and
 * rlk_linear_logp_dh_merge adds slice results by the tree. So dhidden has the
 * same bits at TP = 1, 2 and 4, and every row of dweight (one owner per
 * element, a chain over t) has the same bits in a slice call as in the
 * whole-vocabulary call. Any other call covers one segment starting at its
 * first row.
 */
#ifndef RLK_LINEAR_H
#define RLK_LINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RLK_API __attribute__((visibility("default")))

typedef enum rlk_status {
  RLK_OK = 0,
  RLK_ERR_INVALID_ARG = 1,         /* null/misaligned pointer, negative size, bad range, bad flag */
  RLK_ERR_UNSUPPORTED_SHAPE = 2,   /* H not a positive multiple of 64, or a size beyond the limits */
  RLK_ERR_WORKSPACE_TOO_SMALL = 3, /* workspace_bytes below the matching *_workspace_bytes() */
  RLK_ERR_UNSUPPORTED_DEVICE = 4,  /* the current device is not gfx950 */
  RLK_ERR_HIP = 5,                 /* a HIP runtime call failed (no device, launch failure) */
  RLK_ERR_SCRATCH_LIMIT = 6        /* rlk_linear_logp_fwd_noalloc: records beyond its static scratch */
} rlk_status;

/* Per-row statistics record, 4 floats per row (row-major [T][4]):
 *   m  = max_v z_{t,v} over the covered vocabulary,
 *   R  = sum over the covered vocabulary, without one arg-max entry, of exp(z - m),
 *   B  = sum over the covered vocabulary of exp(z - m) (z - m)   (<= 0),
 *   zy = z_{t,y_t} if y_t is covered, else -inf.
 * Over the whole vocabulary: logp = (zy - m) - log1p(R) and
 * entropy = log1p(R) - B / (1 + R). */
#define RLK_STATS_WIDTH 4

/* bwd flags */
#define RLK_DH_F32 1u /* dhidden is fp32 [T,H] (e.g. one slice's partial); default bf16 */

/* Limits checked by every entry point. T and V (the rows of W in one call)
 * are bounded so that the byte offsets inside any 256-row tile of the
 * kernels' operands fit the 32-bit buffer offsets (RLK_ERR_UNSUPPORTED_SHAPE
 * beyond them); vocab_total is bounded by the int32 target ids
 * (RLK_ERR_INVALID_ARG beyond it). */
#define RLK_MAX_T (1LL << 21)
#define RLK_MAX_H 65536
#define RLK_MAX_V (1LL << 24)
#define RLK_MAX_VOCAB ((1LL << 31) - 1)

/* Source: the rollout side runs the op inside captured CUDA graphs of batch
 * 1-4 (page "RL-Kernel evidence h100-cp-gradient.json",
 * validation.cudagraph.expected_capture_sizes), where nothing may allocate:
 * the caller sizes and owns every scratch buffer.
 * Bytes of device workspace the forward needs for (T, H, V): one 16-byte
 * record per row and group of 256 columns, (ceil(V/256) + 3) groups at most,
 * two records per group (one per 128-column half) when T <= 64, rounded up
 * to 256 bytes. 0 when T == 0. */
RLK_API size_t rlk_linear_logp_fwd_workspace_bytes(int64_t T, int64_t H, int64_t V);

/* Source: the training side differentiates through the op (page "RL-Kernel
 * evidence h100-cp-gradient.json", validation.runtime_readbacks.frameworks
 * ['megatron/training'].modules.logp); its scratch is the caller's, as above.
 * Bytes of device workspace the backward needs for (T, H, V, flags, whether
 * dhidden is requested). 0 when T == 0. */
RLK_API size_t rlk_linear_logp_bwd_workspace_bytes(int64_t T, int64_t H, int64_t V,
                                                   uint32_t flags, int want_dhidden);

/* Forward. Source: the linear-logp provider that stands in for VIME's
 * calculate_log_probs_and_entropy (page "VIME Qwen3-8B TP4/CP2 200-round
 * consistency experiment", section "User-facing operator matrix"), called by
 * both the trainer and the rollout engine with bit-equal results (page
 * "RL-Kernel evidence h100-cp-gradient.json", validation.train_rollout_logprob
 * and validation.runtime_scalar_logprob: 0 bitwise mismatches, max |d| = 0).
 *   hidden   bf16 [T,H]
 *   weight   bf16 [V,H], rows vocab_start .. vocab_start+V-1 of the LM head
 *   targets  int32 [T], global ids; 0 <= y < vocab_total is a precondition
 *            (a row that breaks it gets logp = NaN)
 *   logp, entropy  fp32 [T] or NULL; must be NULL unless the call covers the
 *            whole vocabulary (vocab_start == 0 and V == vocab_total)
 *   stats    fp32 [T,4] or NULL: the record above for the covered vocabulary
 *   workspace, workspace_bytes: >= rlk_linear_logp_fwd_workspace_bytes(T,H,V)
 * T == 0 is a no-op. At least one of logp, entropy, stats must be non-NULL. */
RLK_API rlk_status rlk_linear_logp_fwd(const void* hidden, const void* weight,
                                       const int32_t* targets, int64_t T, int64_t H, int64_t V,
                                       int64_t vocab_start, int64_t vocab_total, float* logp,
                                       float* entropy, float* stats, void* workspace,
                                       size_t workspace_bytes, void* stream);

/* Allocation-free forward, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. Arguments and results as rlk_linear_logp_fwd (the same kernels,
 * so the same bits) without workspace: the records go to a static device
 * array of RLK_NOALLOC_SCRATCH_BYTES that the library holds on each device it
 * runs on until the process ends. Calls whose
 * rlk_linear_logp_fwd_workspace_bytes(T, H, V) exceeds it return
 * RLK_ERR_SCRATCH_LIMIT before anything is launched (8 MiB holds T up to 878
 * rows of a 151,936-row vocabulary, or 64 rows of a 1,000,000-row one).
 * Nothing in the scratch needs to start at zero: every record a result
 * depends on is written by the same call. All calls on one device share that
 * device's scratch, which keeps the last call's records: calls that overlap
 * in time on one device (different streams, or host threads without
 * ordering) race and give undefined results; calls ordered on one stream are
 * safe. The first call on a device looks up the scratch's device address
 * (hipGetSymbolAddress, with that device current) and keeps it. */
#define RLK_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
RLK_API rlk_status rlk_linear_logp_fwd_noalloc(const void* hidden, const void* weight,
                                               const int32_t* targets, int64_t T, int64_t H,
                                               int64_t V, int64_t vocab_start,
                                               int64_t vocab_total, float* logp, float* entropy,
                                               float* stats, void* stream);

/* Packed weight for the streaming forward. Source: the rollout engine scores
 * decode batches of 1-4 rows (page "RL-Kernel evidence h100-cp-gradient.json",
 * validation.cudagraph.expected_capture_sizes; page "VIME Qwen3-8B TP4/CP2
 * 200-round consistency experiment", section "Required gates": CUDA Graph
 * evidence must match) and must return the trainer's bits
 * (validation.train_rollout_logprob).
 *
 * Rollout calls the forward with a few rows at a time (the decode batch) and
 * a weight that stays fixed for the whole rollout, so the forward is a read
 * of W at the HBM rate. In its natural [V,H] layout the library reads W as
 * 64-byte pieces of 128 rows at a time (one MFMA k-step of one 128-row unit);
 * the packed copy holds the same elements in the order the stream consumes
 * them, so each step reads 8 KB that are contiguous, a pattern HBM serves
 * markedly faster. Values, arithmetic and results are identical: the forward
 * over the packed copy returns the same bits as rlk_linear_logp_fwd over W.
 *
 * Layout (for the slicing the forward derives from V, vocab_start and
 * vocab_total: see tensor-parallel invariance above): the call's rows form P
 * slices of Vs rows; unit iu of slice p is slice rows 128 iu .. 128 iu + 127,
 * units numbered pu = p * ceil(Vs/128) + iu, each 128 * H bf16 at offset
 * pu * 128 * H. Inside a unit, k-step s (elements 32 s .. 32 s + 31 of each
 * row) is 4096 bf16 at offset 4096 s; inside a step, 16-byte piece i of
 * 1 KB block b holds row 16 b + r, r = i / 4, and its 8-element piece
 * ((i % 4) - r / 2) mod 4 (integer r / 2). Rows past the
 * slice are zero. The layout is tied to (H, V, vocab_start, vocab_total):
 * pack and use with the same four values. */
RLK_API size_t rlk_linear_pack_weight_bytes(int64_t H, int64_t V, int64_t vocab_start,
                                            int64_t vocab_total);
/* Source: as the size query above (rollout-side scoring, same bits).
 * weight bf16 [V,H] (16-byte aligned); packed: device buffer of packed_bytes >=
 * rlk_linear_pack_weight_bytes(...), 16-byte aligned, written on `stream`.
 * Errors as the forward's shape and argument checks;
 * RLK_ERR_WORKSPACE_TOO_SMALL if packed_bytes is short. */
RLK_API rlk_status rlk_linear_pack_weight(const void* weight, int64_t H, int64_t V,
                                          int64_t vocab_start, int64_t vocab_total, void* packed,
                                          size_t packed_bytes, void* stream);
/* Source: as rlk_linear_logp_fwd_workspace_bytes (no allocation inside a
 * captured rollout graph). Workspace of the packed forward: two 16-byte
 * records per row and group. */
RLK_API size_t rlk_linear_logp_fwd_packed_workspace_bytes(int64_t T, int64_t H, int64_t V);
/* Source: rollout-side scoring with the trainer's bits (page "RL-Kernel
 * evidence h100-cp-gradient.json", validation.runtime_readbacks.frameworks
 * ['vllm/rollout'].modules.logp and validation.train_rollout_logprob).
 * The forward over a packed weight: arguments and results as
 * rlk_linear_logp_fwd, with packed_weight/packed_bytes from
 * rlk_linear_pack_weight for the same (H, V, vocab_start, vocab_total)
 * (RLK_ERR_INVALID_ARG if packed_bytes is short) and the workspace from
 * rlk_linear_logp_fwd_packed_workspace_bytes. Any T works; W is streamed once
 * per 64 rows, so it is meant for T <= 64 (decode batches). */
RLK_API rlk_status rlk_linear_logp_fwd_packed(const void* hidden, const void* packed_weight,
                                              size_t packed_bytes, const int32_t* targets,
                                              int64_t T, int64_t H, int64_t V,
                                              int64_t vocab_start, int64_t vocab_total,
                                              float* logp, float* entropy, float* stats,
                                              void* workspace, size_t workspace_bytes,
                                              void* stream);

/* Backward. Source: the actor-train phase back-propagates through the op
 * (page "RL-Kernel evidence h100-cp-gradient.json",
 * validation.runtime_readbacks.frameworks['megatron/training'].modules.logp),
 * and its gradients must not depend on the parallel layout
 * (gradient_norm_comparisons: exactly_equal between the TP2/CP4 and TP4/CP2
 * runs; all_parameter_hash_comparisons: bitwise_equal).
 *   hidden, weight, targets, T, H, V, vocab_start, vocab_total: as in the forward
 *   stats    fp32 [T,4] whole-vocabulary record (the forward's `stats` for a
 *            full call, or the combined record for slices)
 *   dlogp    fp32 [T] or NULL (= 0)
 *   dentropy fp32 [T] or NULL (= 0)
 *   dhidden  [T,H] bf16 (fp32 with RLK_DH_F32), or NULL to skip. For a slice it
 *            is that slice's contribution sum_{v in slice} G[t,v] W[v,:]
 *            (ask for fp32 and add slices with rlk_linear_logp_dh_merge).
 *   dweight  fp32 [V,H], overwritten, or NULL to skip
 *   flags    0 or RLK_DH_F32
 *   workspace, workspace_bytes: >= rlk_linear_logp_bwd_workspace_bytes(
 *            T, H, V, flags, dhidden != NULL)
 * G[t,v] = dlogp_t ([v == y_t] - p_{t,v}) - dentropy_t p_{t,v} (log p_{t,v} + entropy_t).
 * T == 0 with dweight != NULL writes zeros to dweight. */
RLK_API rlk_status rlk_linear_logp_bwd(const void* hidden, const void* weight,
                                       const int32_t* targets, int64_t T, int64_t H, int64_t V,
                                       int64_t vocab_start, int64_t vocab_total,
                                       const float* stats, const float* dlogp,
                                       const float* dentropy, void* dhidden, float* dweight,
                                       uint32_t flags, void* workspace, size_t workspace_bytes,
                                       void* stream);

/* Source: the actor runs the LM head at TP=4 (page "VIME Qwen3-8B TP4/CP2
 * 200-round consistency experiment", section "Required gates"), and the
 * TP2/CP4 and TP4/CP2 runs agree bit for bit (page "RL-Kernel evidence
 * h100-cp-gradient.json", gradient_norm_comparisons,
 * all_parameter_hash_comparisons), so slice records merge in an order that
 * does not depend on the TP degree.
 * Merge of S slice records (slices in vocabulary order) by the fixed merge
 * tree: adjacent pairs first, (r0 + r1), (r2 + r3), ..., an odd last record
 * carried up unchanged, repeated until one record is left; so S = 2 gives
 * r0 + r1 and S = 4 gives (r0 + r1) + (r2 + r3).
 *   partials  fp32 [S][T][4] (slice s's forward `stats`), 1 <= S <= 1024
 *   logp, entropy  fp32 [T] or NULL (a row whose target lies in no slice
 *            gets logp = -inf)
 *   stats     fp32 [T,4] or NULL: the merged whole-vocabulary record
 * rlk_linear_logp_combine takes device pointers and runs on `stream` with the
 * arithmetic of the forward kernels, so its bits equal those of a call that
 * covers the same slices (see "Tensor-parallel invariance"); at least one
 * output must be non-NULL, T == 0 is a no-op.
 * rlk_linear_logp_combine_host takes host pointers and runs on the CPU
 * (touches no device); its exp and log1p are the host library's, so its
 * values agree with the device's to rounding but not necessarily in every
 * bit. */
RLK_API rlk_status rlk_linear_logp_combine(const float* partials, int64_t S, int64_t T,
                                           float* logp, float* entropy, float* stats,
                                           void* stream);
RLK_API rlk_status rlk_linear_logp_combine_host(const float* partials, int64_t S, int64_t T,
                                                float* logp, float* entropy, float* stats);

/* Source: as rlk_linear_logp_combine (actor at TP=4; gradient_norm_comparisons
 * exactly_equal across parallel layouts).
 * Sum of S fp32 dH contributions of slice calls (slices in vocabulary order,
 * each from rlk_linear_logp_bwd with RLK_DH_F32) by the fixed merge tree of
 * rlk_linear_logp_combine (S = 2: p0 + p1; S = 4: (p0 + p1) + (p2 + p3)),
 * then bf16 round-to-nearest-even into dhidden, or fp32 with RLK_DH_F32.
 * With the slice calls of a TP = 2 or 4 layout it returns the bits of the
 * whole-vocabulary backward's dhidden.
 *   parts    fp32 [S][T][H] device, 1 <= S <= 1024
 *   dhidden  [T,H] bf16 (fp32 with RLK_DH_F32) device
 * H a positive multiple of 64 (RLK_ERR_UNSUPPORTED_SHAPE otherwise); T == 0
 * is a no-op. Runs on `stream`. */
RLK_API rlk_status rlk_linear_logp_dh_merge(const float* parts, int64_t S, int64_t T, int64_t H,
                                            void* dhidden, uint32_t flags, void* stream);

/* Source: strict mode fails on any fallback (page "RL-Kernel
 * h3-runtime-integration-b200 report.json", runtime_modes.strict:
 * fail_on_fallback) and R/R runs must show no fallback provenance (page "VIME
 * Qwen3-8B TP4/CP2 200-round consistency experiment", section "Required
 * gates"): every failure is a status code, never a silent other route.
 * Text of a status code. */
RLK_API const char* rlk_status_string(int status);
/* Source: the runtime reads back, per framework and module, the backend ids
 * and call counts that ran (page "RL-Kernel evidence h100-cp-gradient.json",
 * validation.runtime_readbacks: backend_ids, call_count).
 * Backend id of this library ("rlk.linear_logp.bitwise.gfx950.v1"). */
RLK_API const char* rlk_backend_id(void);
/* Source: as rlk_backend_id (validation.runtime_readbacks: call_count).
 * Number of successful calls since load: which = 0 fwd, 1 bwd, 2 combine_host,
 * 3 combine, 4 pack_weight, 5 fwd_packed, 6 fwd_noalloc, 7 dh_merge. */
RLK_API uint64_t rlk_call_count(int which);
/* Source: as rlk_backend_id (the readback names the exact backend version).
 * Version of this ABI (1). */
RLK_API int rlk_abi_version(void);

/* Source: the pages time the log-prob pass per phase (page "RL-Kernel
 * evidence h100-cp-gradient.json", runs[].performance: perf/log_probs_time,
 * perf/actor_train_time); this timer splits such a pass per kernel.
 * Per-launch event timer, for measurement. After rlk_profile_begin every
 * kernel launch of the library is bracketed by two HIP events recorded on the
 * launch's own stream (launch order and work are unchanged).
 * rlk_profile_end waits for those events, stops the timer and writes, per
 * kernel id in [0, n), the summed elapsed milliseconds and the number of
 * launches (host arrays of n entries; n = rlk_profile_kernel_count() covers
 * every kernel). Returns RLK_ERR_HIP if an event could not be created,
 * recorded or read. Not thread-safe against concurrent begin/end. */
RLK_API rlk_status rlk_profile_begin(void);
RLK_API rlk_status rlk_profile_end(double* total_ms, uint64_t* launches, int n);
RLK_API int rlk_profile_kernel_count(void);
RLK_API const char* rlk_profile_kernel_name(int id);

#ifdef __cplusplus
}
#endif

#endif /* RLK_LINEAR_H */
