// rlk_internal.h — host-side plan and launcher interface between the C ABI
// (rlk_abi.cpp) and the kernels (rlk_kernels.hip). Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rlk {

// Batches of at most this many rows run the forward as a stream over W
// (fwd_stream_kernel) and the backward on 32-row tiles; larger ones run
// 256-row tiles. All of them compute each logit by the same MFMA chain and
// each record by the same reduction order, so a row's bits do not depend on
// which one ran.
constexpr int kSmallT = 64;

// dH is reduced over fixed vocabulary splits, about one per kSplitCols
// columns of a virtual slice (at most kMaxSplits in a call), each a multiple
// of 256 columns and starting at its slice's first row.
constexpr int kMaxSplits = 8;
constexpr int kSplitCols = 16384;
// Soft bound on the elements of one bf16 logit-gradient chunk (T x columns).
constexpr int64_t kChunkElems = int64_t(1) << 28;
// A chunk of G at most this large stays in the 256 MB Infinity Cache between
// the recompute that writes it and dW and dH that read it, if the recompute's
// stream of W does not push it out: the recompute then loads W non-temporal.
constexpr size_t kGResidentBytes = size_t(192) << 20;
// Columns h of one dW tile (the tile is 256 v x kDwBN h).
constexpr int kDwBN = 128;

// Assignment of dW tiles to XCDs: `groups` sets of XCDs, each owning
// h_per_group h-tiles; the 8 / groups XCDs of a set split the v-tiles,
// v_per_xcd each; per_xcd workgroups per XCD.
struct DwMap {
  int groups, h_per_group, v_per_xcd, per_xcd;
};
DwMap dw_map(int n_vtiles, int n_htiles);

// The splits of the backward, as the kernels see them: P virtual slices of Vs
// rows, padded to Vs_pad columns, each cut into n_sub splits of split_w
// columns from the slice's first row (the last one shorter).
struct SplitMap {
  int Vs, Vs_pad, n_sub, split_w;
};

// Forward reduction layout. With P > 1 the call covers P of the 4 virtual
// slices (vocab_total / 4 rows each) of the vocabulary: groups of 256
// columns restart at each slice's first row (Gs groups per slice, the last
// one short), each slice is reduced on its own, and the slice records merge
// by the fixed tree. Otherwise P = 1 and the one segment is the call.
constexpr int kVirtualSlices = 4;
struct FwdSlicing {
  int P;       // virtual slices covered by the call (1, 2 or 4)
  int Vs;      // rows per slice
  int Gs;      // groups per slice
  int G;       // P * Gs
  int sliced;  // 1 when the call follows the virtual slices (vocab_total / 4 rows each)
};
FwdSlicing fwd_slicing(int64_t V, int64_t vocab_start, int64_t vocab_total);
// Records merged by one combine call, and the depth of its merge stack.
constexpr int kMaxCombine = 1024;
constexpr int kCombineDepth = 12;

struct FwdArgs {
  const uint16_t* hidden;
  const uint16_t* weight;
  const int32_t* targets;
  int T, H, V;
  int64_t vocab_start, vocab_total;
  int full;
  FwdSlicing slicing;
  int n_cu;    // compute units of the device (persistent small-batch grid)
  int packed;  // weight is the pack_weight layout (fwd_stream only)
  float* logp;
  float* entropy;
  float4* stats;
  float4* part;  // workspace [T][G]
};

// Backward vocabulary layout. The call's rows form P virtual slices of Vs
// rows (the forward's slicing). Each slice is cut into n_sub splits of
// split_w columns (a multiple of 256, the last one shorter) from the slice's
// first row; n_sub depends on Vs alone, so a call at TP = 1, 2 or 4 cuts every
// virtual slice the same way. The logit gradient, the recompute tiles and the
// dW tiles live in the padded layout: column u is row u % Vs_pad of slice
// u / Vs_pad (Vs_pad = Vs rounded up to 256), and the columns past a slice's
// end hold zeros. dH of a row is the sum over each slice's splits in order,
// then the slices by the fixed tree ((s0 + s1) + (s2 + s3)).
struct BwdPlan {
  int P, Vs, Vs_pad;    // virtual slices of the call, rows per slice, padded
  int n_sub;            // splits per slice
  int split_w;          // columns per split (multiple of 256)
  int nsplits;          // P * n_sub
  int splits_per_chunk;
  int nchunks;
  int64_t ldg;          // row stride of the G chunk buffer (columns)
  int64_t Tp;           // T rounded up to the dW k-step (32)
  size_t off_gtv, off_part, total;
  // padded column where split s begins / ends, and its valid columns
  int u_begin(int s) const { return (s / n_sub) * Vs_pad + (s % n_sub) * split_w; }
  int u_end(int s) const {
    const int e = (s % n_sub + 1) * split_w;
    return (s / n_sub) * Vs_pad + (e < Vs_pad ? e : Vs_pad);
  }
  int split_len(int s) const {
    const int r = Vs - (s % n_sub) * split_w;
    return r < split_w ? r : split_w;
  }
};

struct BwdArgs {
  const uint16_t* hidden;
  const uint16_t* weight;
  const int32_t* targets;
  int T, H, V;
  int64_t vocab_start, vocab_total;
  const float4* stats;
  const float* dlogp;
  const float* dentropy;
  void* dhidden;
  int dh_f32;
  float* dweight;
  uint16_t* gtv;  // [Tp][ldg] logit gradient of one chunk, rows t (dH and dW operand)
  float* part;
  int n_cu;  // compute units of the device (persistent recompute grid)
};

// Kernel ids for the optional per-launch event timer (rlk_profile_*).
enum KernelId {
  K_FWD_TILE = 0,
  K_FWD_COMBINE,
  K_BWD_RECOMPUTE,
  K_BWD_DW,
  K_BWD_DH,
  K_BWD_DH_REDUCE,
  K_FILL_ZERO,
  K_COMBINE,
  K_FWD_STREAM,
  K_PACK,
  K_DH_MERGE,
  K_COUNT
};
extern const char* const kKernelNames[K_COUNT];
// Record a HIP event on `st` before / after a launch of kernel `id`; no-ops
// unless the timer is on.
void prof_before(int id, hipStream_t st);
void prof_after(int id, hipStream_t st);

size_t fwd_workspace(int64_t T, int64_t H, int64_t V, bool packed);
size_t packed_weight_bytes(int64_t H, const FwdSlicing& sl);
hipError_t launch_pack(const uint16_t* weight, int H, const FwdSlicing& sl, uint16_t* packed,
                       hipStream_t st);
// RLK_OK when the current device is gfx950, else the rlk_status error.
int check_device_status();
BwdPlan bwd_plan(int64_t T, int64_t H, const FwdSlicing& sl, bool want_dh);
// Workspace bytes that cover a backward of (T, H, V) under any slicing.
size_t bwd_workspace_any(int64_t T, int64_t H, int64_t V, bool want_dh);

hipError_t launch_fwd(const FwdArgs& a, hipStream_t st);
hipError_t launch_bwd(const BwdArgs& a, const BwdPlan& p, hipStream_t st);
hipError_t launch_combine(const float4* partials, int S, int T, float* logp, float* entropy,
                          float4* stats, hipStream_t st);
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t st);
hipError_t launch_dh_merge(const float* parts, int S, int64_t n, int out_f32, void* out,
                           hipStream_t st);

}  // namespace rlk
