// rlk_abi.cpp — the C ABI of the linear log-prob library: argument checks,
// workspace planning, device check, launch sequencing, host-side combine and
// provenance. Every argument error is returned before any HIP call.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>
#include <vector>

#include "rlk_internal.h"
#include "../../include/rlk_linear.h"

namespace {

constexpr int kAbiVersion = 1;
const char kBackendId[] = "rlk.linear_logp.bitwise.gfx950.v1";

std::atomic<uint64_t> g_calls[8];

// Scratch of rlk_linear_logp_fwd_noalloc: the forward's per-(row, group)
// record buffer, in device memory that the code object itself holds (one
// copy per device, from module load until the process ends), so that the
// entry point allocates nothing. In host code `scratch` is only a stand-in
// for the symbol, never a device address: kernels and copies get the address
// that hipGetSymbolAddress returns for the current device.
constexpr size_t kScratchBytes = RLK_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 256;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
rlk_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return RLK_ERR_HIP;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return RLK_ERR_HIP;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return RLK_OK;
}

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
inline int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Shape checks shared by fwd and bwd.
rlk_status check_shape(int64_t T, int64_t H, int64_t V, int64_t vocab_start, int64_t vocab_total) {
  if (T < 0 || H <= 0 || V <= 0 || vocab_start < 0 || vocab_total <= 0) return RLK_ERR_INVALID_ARG;
  if (vocab_total > RLK_MAX_VOCAB || V > vocab_total || vocab_start > vocab_total - V)
    return RLK_ERR_INVALID_ARG;
  if (T > RLK_MAX_T || H > RLK_MAX_H || V > RLK_MAX_V || (H % 64) != 0)
    return RLK_ERR_UNSUPPORTED_SHAPE;
  return RLK_OK;
}

// The kernels are built for gfx950 only; refuse anything else. On success
// *n_cu (if given) receives the current device's compute-unit count.
rlk_status check_device(int* n_cu = nullptr) {
  static std::atomic<int> cache[256];  // 0 unknown, 1 gfx950, 2 other
  static std::atomic<int> cus[256];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return RLK_ERR_HIP;
  if (dev < 256) {
    const int c = cache[dev].load(std::memory_order_acquire);
    if (c == 2) return RLK_ERR_UNSUPPORTED_DEVICE;
    if (c == 1) {
      if (n_cu) *n_cu = cus[dev].load(std::memory_order_relaxed);
      return RLK_OK;
    }
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return RLK_ERR_HIP;
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  const int ncu = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 0;
  if (dev < 256) {
    cus[dev].store(ncu, std::memory_order_relaxed);
    cache[dev].store(ok ? 1 : 2, std::memory_order_release);
  }
  if (ok && n_cu) *n_cu = ncu;
  return ok ? RLK_OK : RLK_ERR_UNSUPPORTED_DEVICE;
}

// Per-launch event timer: while on, every launch is bracketed by two HIP
// events on its stream; rlk_profile_end sums the elapsed times per kernel.
struct Profiler {
  std::atomic<bool> on{false};
  std::mutex mu;
  struct Rec {
    int id;
    hipEvent_t a, b;
  };
  std::vector<Rec> recs;
  std::vector<hipEvent_t> pool;
  size_t next = 0;
  bool failed = false;

  hipEvent_t take() {
    if (next == pool.size()) {
      hipEvent_t e = nullptr;
      if (hipEventCreate(&e) != hipSuccess) {
        failed = true;
        return nullptr;
      }
      pool.push_back(e);
    }
    return pool[next++];
  }
};
Profiler g_prof;

}  // namespace

namespace rlk {

int check_device_status() { return (int)check_device(); }

const char* const kKernelNames[K_COUNT] = {
    "fwd_tile",      "fwd_combine", "bwd_recompute", "bwd_dw",      "bwd_dh",
    "bwd_dh_reduce", "fill_zero",   "combine",       "fwd_stream",  "pack_weight", "dh_merge"};

void prof_before(int id, hipStream_t st) {
  if (!g_prof.on.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lk(g_prof.mu);
  hipEvent_t e = g_prof.take();
  if (!e) return;
  if (hipEventRecord(e, st) != hipSuccess) {
    g_prof.failed = true;
    return;
  }
  g_prof.recs.push_back({id, e, nullptr});
}

void prof_after(int id, hipStream_t st) {
  if (!g_prof.on.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lk(g_prof.mu);
  if (g_prof.recs.empty() || g_prof.recs.back().id != id || g_prof.recs.back().b) return;
  hipEvent_t e = g_prof.take();
  if (!e) return;
  if (hipEventRecord(e, st) != hipSuccess) {
    g_prof.failed = true;
    return;
  }
  g_prof.recs.back().b = e;
}

size_t fwd_workspace(int64_t T, int64_t H, int64_t V, bool packed) {
  (void)H;
  if (T <= 0) return 0;
  // P virtual slices of V / P rows take at most ceil(V/256) + P - 1 groups;
  // the stream path keeps one record per 128-column half of a group
  const int64_t G = ceil_div(V, 256) + kVirtualSlices - 1;
  return align256(size_t(T) * size_t(G) * (packed || T <= kSmallT ? 2 : 1) * 16);
}

size_t packed_weight_bytes(int64_t H, const FwdSlicing& sl) {
  return size_t(sl.P) * size_t(ceil_div(sl.Vs, 128)) * 128 * size_t(H) * 2;
}

FwdSlicing fwd_slicing(int64_t V, int64_t vocab_start, int64_t vocab_total) {
  FwdSlicing f{1, (int)V, 0, 0, 0};
  if (vocab_total % kVirtualSlices == 0) {
    const int64_t vs = vocab_total / kVirtualSlices;
    if (vocab_start % vs == 0 && V % vs == 0) {
      const int64_t p = V / vs, first = vocab_start / vs;
      if ((p == 1 || p == 2 || p == 4) && first % p == 0) {
        f.P = (int)p;
        f.Vs = (int)vs;
        f.sliced = 1;
      }
    }
  }
  f.Gs = (int)ceil_div(f.Vs, 256);
  f.G = f.P * f.Gs;
  return f;
}

BwdPlan bwd_plan(int64_t T, int64_t H, const FwdSlicing& sl, bool want_dh) {
  BwdPlan p{};
  p.P = sl.P;
  p.Vs = sl.Vs;
  p.Vs_pad = (int)round_up(sl.Vs, 256);
  // splits per slice: from the slice size alone (and, for the virtual slices,
  // a cap that keeps 4 slices within kMaxSplits)
  int64_t S = sl.Vs / kSplitCols;
  const int64_t cap = sl.sliced ? kMaxSplits / kVirtualSlices : kMaxSplits;
  if (S < 1) S = 1;
  if (S > cap) S = cap;
  p.split_w = (int)round_up(ceil_div(p.Vs_pad, S), 256);
  p.n_sub = (int)ceil_div(p.Vs_pad, p.split_w);
  p.nsplits = p.P * p.n_sub;
  // dW walks K = t over [0, Tp) in steps of 32 (rows t >= T read as zero)
  p.Tp = round_up(T > 0 ? T : 1, 32);
  int64_t spc = kChunkElems / (p.Tp * p.split_w);
  if (spc < 1) spc = 1;
  if (spc > p.nsplits) spc = p.nsplits;
  p.splits_per_chunk = (int)spc;
  p.nchunks = (int)ceil_div(p.nsplits, spc);
  p.ldg = spc * p.split_w;
  p.off_gtv = 0;
  p.off_part = align256(p.off_gtv + size_t(p.Tp) * size_t(p.ldg) * 2);
  p.total = align256(p.off_part + (want_dh ? size_t(p.nsplits) * size_t(T) * size_t(H) * 4 : 0));
  return p;
}

size_t bwd_workspace_any(int64_t T, int64_t H, int64_t V, bool want_dh) {
  // the unsliced layout, and V as 1, 2 or 4 virtual slices
  const FwdSlicing whole{1, (int)V, 0, 0, 0};
  size_t m = bwd_plan(T, H, whole, want_dh).total;
  for (int P : {1, 2, 4}) {
    if (V % P != 0) continue;
    const FwdSlicing sl{P, (int)(V / P), 0, 0, 1};
    const size_t t = bwd_plan(T, H, sl, want_dh).total;
    m = t > m ? t : m;
  }
  return m;
}

}  // namespace rlk

extern "C" {

RLK_API size_t rlk_linear_logp_fwd_workspace_bytes(int64_t T, int64_t H, int64_t V) {
  if (T <= 0 || H <= 0 || V <= 0) return 0;
  return rlk::fwd_workspace(T, H, V, false);
}

RLK_API size_t rlk_linear_logp_fwd_packed_workspace_bytes(int64_t T, int64_t H, int64_t V) {
  if (T <= 0 || H <= 0 || V <= 0) return 0;
  return rlk::fwd_workspace(T, H, V, true);
}

RLK_API size_t rlk_linear_pack_weight_bytes(int64_t H, int64_t V, int64_t vocab_start,
                                            int64_t vocab_total) {
  if (check_shape(0, H, V, vocab_start, vocab_total) != RLK_OK) return 0;
  return rlk::packed_weight_bytes(H, rlk::fwd_slicing(V, vocab_start, vocab_total));
}

RLK_API rlk_status rlk_linear_pack_weight(const void* weight, int64_t H, int64_t V,
                                          int64_t vocab_start, int64_t vocab_total, void* packed,
                                          size_t packed_bytes, void* stream) {
  rlk_status s = check_shape(0, H, V, vocab_start, vocab_total);
  if (s != RLK_OK) return s;
  if (!weight || !aligned(weight, 16) || !packed || !aligned(packed, 16)) return RLK_ERR_INVALID_ARG;
  const rlk::FwdSlicing sl = rlk::fwd_slicing(V, vocab_start, vocab_total);
  if (packed_bytes < rlk::packed_weight_bytes(H, sl)) return RLK_ERR_WORKSPACE_TOO_SMALL;
  s = check_device();
  if (s != RLK_OK) return s;
  if (rlk::launch_pack(static_cast<const uint16_t*>(weight), (int)H, sl,
                       static_cast<uint16_t*>(packed), static_cast<hipStream_t>(stream)) != hipSuccess)
    return RLK_ERR_HIP;
  g_calls[4].fetch_add(1, std::memory_order_relaxed);
  return RLK_OK;
}

RLK_API size_t rlk_linear_logp_bwd_workspace_bytes(int64_t T, int64_t H, int64_t V,
                                                   uint32_t flags, int want_dhidden) {
  (void)flags;
  if (T <= 0 || H <= 0 || V <= 0) return 0;
  return rlk::bwd_workspace_any(T, H, V, want_dhidden != 0);
}

namespace {
// The forward for the natural layout (packed_bytes == 0) or the packed one;
// with noalloc the records go to the static scratch instead of the caller's
// workspace.
rlk_status fwd_call(const void* hidden, const void* weight, bool packed, size_t packed_bytes,
                    const int32_t* targets, int64_t T, int64_t H, int64_t V, int64_t vocab_start,
                    int64_t vocab_total, float* logp, float* entropy, float* stats,
                    void* workspace, size_t workspace_bytes, void* stream, bool noalloc = false) {
  const int counter = noalloc ? 6 : packed ? 5 : 0;

  rlk_status s = check_shape(T, H, V, vocab_start, vocab_total);
  if (s != RLK_OK) return s;
  const bool full = vocab_start == 0 && V == vocab_total;
  if (!full && (logp || entropy)) return RLK_ERR_INVALID_ARG;
  if (!logp && !entropy && !stats) return RLK_ERR_INVALID_ARG;
  if (!weight || !aligned(weight, 16)) return RLK_ERR_INVALID_ARG;
  if (T == 0) {
    g_calls[counter].fetch_add(1, std::memory_order_relaxed);
    return RLK_OK;
  }
  if (!hidden || !aligned(hidden, 16) || !targets || !aligned(targets, 4)) return RLK_ERR_INVALID_ARG;
  if ((logp && !aligned(logp, 4)) || (entropy && !aligned(entropy, 4)) ||
      (stats && !aligned(stats, 16)))
    return RLK_ERR_INVALID_ARG;
  if (packed &&
      packed_bytes < rlk::packed_weight_bytes(H, rlk::fwd_slicing(V, vocab_start, vocab_total)))
    return RLK_ERR_INVALID_ARG;
  const size_t need = rlk::fwd_workspace(T, H, V, packed);
  if (noalloc) {
    if (need > kScratchBytes) return RLK_ERR_SCRATCH_LIMIT;
  } else {
    if (workspace_bytes < need) return RLK_ERR_WORKSPACE_TOO_SMALL;
    if (!workspace || !aligned(workspace, 16)) return RLK_ERR_INVALID_ARG;
  }
  int n_cu = 0;
  s = check_device(&n_cu);
  if (s != RLK_OK) return s;
  if (noalloc) {
    s = scratch_address(&workspace);
    if (s != RLK_OK) return s;
  }

  rlk::FwdArgs a{};
  a.n_cu = n_cu;
  a.packed = packed ? 1 : 0;
  a.hidden = static_cast<const uint16_t*>(hidden);
  a.weight = static_cast<const uint16_t*>(weight);
  a.targets = targets;
  a.T = (int)T;
  a.H = (int)H;
  a.V = (int)V;
  a.vocab_start = vocab_start;
  a.vocab_total = vocab_total;
  a.full = full ? 1 : 0;
  a.slicing = rlk::fwd_slicing(V, vocab_start, vocab_total);
  a.logp = logp;
  a.entropy = entropy;
  a.stats = reinterpret_cast<float4*>(stats);
  a.part = static_cast<float4*>(workspace);
  if (rlk::launch_fwd(a, static_cast<hipStream_t>(stream)) != hipSuccess) return RLK_ERR_HIP;
  g_calls[counter].fetch_add(1, std::memory_order_relaxed);
  return RLK_OK;
}
}  // namespace

RLK_API rlk_status rlk_linear_logp_fwd(const void* hidden, const void* weight,
                                       const int32_t* targets, int64_t T, int64_t H, int64_t V,
                                       int64_t vocab_start, int64_t vocab_total, float* logp,
                                       float* entropy, float* stats, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  return fwd_call(hidden, weight, false, 0, targets, T, H, V, vocab_start, vocab_total, logp,
                  entropy, stats, workspace, workspace_bytes, stream);
}

RLK_API rlk_status rlk_linear_logp_fwd_noalloc(const void* hidden, const void* weight,
                                               const int32_t* targets, int64_t T, int64_t H,
                                               int64_t V, int64_t vocab_start,
                                               int64_t vocab_total, float* logp, float* entropy,
                                               float* stats, void* stream) {
  return fwd_call(hidden, weight, false, 0, targets, T, H, V, vocab_start, vocab_total, logp,
                  entropy, stats, nullptr, 0, stream, true);
}

RLK_API rlk_status rlk_linear_logp_fwd_packed(const void* hidden, const void* packed_weight,
                                              size_t packed_bytes, const int32_t* targets,
                                              int64_t T, int64_t H, int64_t V,
                                              int64_t vocab_start, int64_t vocab_total,
                                              float* logp, float* entropy, float* stats,
                                              void* workspace, size_t workspace_bytes,
                                              void* stream) {
  return fwd_call(hidden, packed_weight, true, packed_bytes, targets, T, H, V, vocab_start,
                  vocab_total, logp, entropy, stats, workspace, workspace_bytes, stream);
}



RLK_API rlk_status rlk_linear_logp_bwd(const void* hidden, const void* weight,
                                       const int32_t* targets, int64_t T, int64_t H, int64_t V,
                                       int64_t vocab_start, int64_t vocab_total,
                                       const float* stats, const float* dlogp,
                                       const float* dentropy, void* dhidden, float* dweight,
                                       uint32_t flags, void* workspace, size_t workspace_bytes,
                                       void* stream) {
  rlk_status s = check_shape(T, H, V, vocab_start, vocab_total);
  if (s != RLK_OK) return s;
  if (flags & ~uint32_t(RLK_DH_F32)) return RLK_ERR_INVALID_ARG;
  if (!weight || !aligned(weight, 16)) return RLK_ERR_INVALID_ARG;
  if (!dhidden && !dweight) return RLK_ERR_INVALID_ARG;
  if (dweight && !aligned(dweight, 16)) return RLK_ERR_INVALID_ARG;
  if (T == 0) {
    if (dweight) {
      s = check_device();
      if (s != RLK_OK) return s;
      if (rlk::launch_fill_zero(dweight, V * H, static_cast<hipStream_t>(stream)) != hipSuccess)
        return RLK_ERR_HIP;
    }
    g_calls[1].fetch_add(1, std::memory_order_relaxed);
    return RLK_OK;
  }
  if (!hidden || !aligned(hidden, 16) || !targets || !aligned(targets, 4)) return RLK_ERR_INVALID_ARG;
  if (!stats || !aligned(stats, 16)) return RLK_ERR_INVALID_ARG;
  if ((dlogp && !aligned(dlogp, 4)) || (dentropy && !aligned(dentropy, 4)))
    return RLK_ERR_INVALID_ARG;
  if (dhidden && !aligned(dhidden, 16)) return RLK_ERR_INVALID_ARG;
  const rlk::FwdSlicing sl = rlk::fwd_slicing(V, vocab_start, vocab_total);
  const rlk::BwdPlan plan = rlk::bwd_plan(T, H, sl, dhidden != nullptr);
  if (workspace_bytes < plan.total) return RLK_ERR_WORKSPACE_TOO_SMALL;
  if (!workspace || !aligned(workspace, 256)) return RLK_ERR_INVALID_ARG;
  int n_cu = 0;
  s = check_device(&n_cu);
  if (s != RLK_OK) return s;

  char* ws = static_cast<char*>(workspace);
  rlk::BwdArgs a{};
  a.n_cu = n_cu;
  a.hidden = static_cast<const uint16_t*>(hidden);
  a.weight = static_cast<const uint16_t*>(weight);
  a.targets = targets;
  a.T = (int)T;
  a.H = (int)H;
  a.V = (int)V;
  a.vocab_start = vocab_start;
  a.vocab_total = vocab_total;
  a.stats = reinterpret_cast<const float4*>(stats);
  a.dlogp = dlogp;
  a.dentropy = dentropy;
  a.dhidden = dhidden;
  a.dh_f32 = (flags & RLK_DH_F32) ? 1 : 0;
  a.dweight = dweight;
  a.gtv = reinterpret_cast<uint16_t*>(ws + plan.off_gtv);
  a.part = reinterpret_cast<float*>(ws + plan.off_part);
  if (rlk::launch_bwd(a, plan, static_cast<hipStream_t>(stream)) != hipSuccess) return RLK_ERR_HIP;
  g_calls[1].fetch_add(1, std::memory_order_relaxed);
  return RLK_OK;
}

// Host merge of slice records, s = 0, 1, ..., S-1 left to right, with the
// same algebra as the device: the larger max is the base (the left one on a
// tie), d = m_other - m_base, R = R_b + e^d (1 + R_o),
// B = B_b + e^d (B_o + (1 + R_o) d), zy = max(zy_1, zy_2).
RLK_API rlk_status rlk_linear_logp_combine_host(const float* partials, int64_t S, int64_t T,
                                                float* logp, float* entropy, float* stats) {
  if (S < 1 || S > rlk::kMaxCombine || T < 0) return RLK_ERR_INVALID_ARG;
  if (T > 0 && !partials) return RLK_ERR_INVALID_ARG;
  struct Rec {
    float m, R, B, zy;
  };
  auto merge = [](const Rec& l, const Rec& r) {
    const bool left_base = !(r.m > l.m);
    const Rec& b = left_base ? l : r;
    const Rec& o = left_base ? r : l;
    Rec out{b.m, b.R, b.B, std::fmax(l.zy, r.zy)};
    if (o.m == -INFINITY) return out;
    const float d = o.m - b.m;
    const float e = std::exp(d);
    const float one_r = 1.f + o.R;
    out.R = b.R + e * one_r;
    out.B = b.B + e * (o.B + one_r * d);
    return out;
  };
  for (int64_t t = 0; t < T; ++t) {
    // the merge tree as a binary counter: a stack of subtrees whose sizes are
    // decreasing powers of two; equal neighbours merge (left + right), and
    // what remains at the end is folded from the right
    Rec st[rlk::kCombineDepth];
    int lvl[rlk::kCombineDepth];
    int n = 0;
    for (int64_t s = 0; s < S; ++s) {
      const float* q = partials + (s * T + t) * 4;
      st[n] = Rec{q[0], q[1], q[2], q[3]};
      lvl[n++] = 0;
      while (n >= 2 && lvl[n - 2] == lvl[n - 1]) {
        st[n - 2] = merge(st[n - 2], st[n - 1]);
        ++lvl[n - 2];
        --n;
      }
    }
    Rec acc = st[n - 1];
    for (int i = n - 2; i >= 0; --i) acc = merge(st[i], acc);
    const float L = std::log1p(acc.R);
    if (stats) {
      stats[t * 4 + 0] = acc.m;
      stats[t * 4 + 1] = acc.R;
      stats[t * 4 + 2] = acc.B;
      stats[t * 4 + 3] = acc.zy;
    }
    if (logp) logp[t] = (acc.zy - acc.m) - L;
    if (entropy) entropy[t] = L - acc.B / (1.f + acc.R);
  }
  g_calls[2].fetch_add(1, std::memory_order_relaxed);
  return RLK_OK;
}

RLK_API rlk_status rlk_linear_logp_combine(const float* partials, int64_t S, int64_t T,
                                           float* logp, float* entropy, float* stats,
                                           void* stream) {
  if (S < 1 || S > rlk::kMaxCombine || T < 0 || T > RLK_MAX_T) return RLK_ERR_INVALID_ARG;
  if (!logp && !entropy && !stats) return RLK_ERR_INVALID_ARG;
  if (T == 0) {
    g_calls[3].fetch_add(1, std::memory_order_relaxed);
    return RLK_OK;
  }
  if (!partials || !aligned(partials, 16) || (logp && !aligned(logp, 4)) ||
      (entropy && !aligned(entropy, 4)) || (stats && !aligned(stats, 16)))
    return RLK_ERR_INVALID_ARG;
  const rlk_status s = check_device();
  if (s != RLK_OK) return s;
  if (rlk::launch_combine(reinterpret_cast<const float4*>(partials), (int)S, (int)T, logp, entropy,
                          reinterpret_cast<float4*>(stats),
                          static_cast<hipStream_t>(stream)) != hipSuccess)
    return RLK_ERR_HIP;
  g_calls[3].fetch_add(1, std::memory_order_relaxed);
  return RLK_OK;
}

RLK_API rlk_status rlk_linear_logp_dh_merge(const float* parts, int64_t S, int64_t T, int64_t H,
                                            void* dhidden, uint32_t flags, void* stream) {
  if (S < 1 || S > rlk::kMaxCombine || T < 0 || H <= 0) return RLK_ERR_INVALID_ARG;
  if (flags & ~uint32_t(RLK_DH_F32)) return RLK_ERR_INVALID_ARG;
  if (T > RLK_MAX_T || H > RLK_MAX_H || (H % 64) != 0) return RLK_ERR_UNSUPPORTED_SHAPE;
  if (T == 0) {
    g_calls[7].fetch_add(1, std::memory_order_relaxed);
    return RLK_OK;
  }
  if (!parts || !aligned(parts, 16) || !dhidden || !aligned(dhidden, 16)) return RLK_ERR_INVALID_ARG;
  const rlk_status s = check_device();
  if (s != RLK_OK) return s;
  if (rlk::launch_dh_merge(parts, (int)S, T * H, (flags & RLK_DH_F32) ? 1 : 0, dhidden,
                           static_cast<hipStream_t>(stream)) != hipSuccess)
    return RLK_ERR_HIP;
  g_calls[7].fetch_add(1, std::memory_order_relaxed);
  return RLK_OK;
}

RLK_API const char* rlk_status_string(int status) {
  switch (status) {
    case RLK_OK: return "ok";
    case RLK_ERR_INVALID_ARG: return "invalid argument";
    case RLK_ERR_UNSUPPORTED_SHAPE: return "unsupported shape (H must be a positive multiple of 64 within the limits)";
    case RLK_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case RLK_ERR_UNSUPPORTED_DEVICE: return "unsupported device (gfx950 required)";
    case RLK_ERR_HIP: return "HIP runtime error";
    case RLK_ERR_SCRATCH_LIMIT:
      return "records exceed the static scratch of rlk_linear_logp_fwd_noalloc "
             "(RLK_NOALLOC_SCRATCH_BYTES); use rlk_linear_logp_fwd with a workspace";
    default: return "unknown status";
  }
}

RLK_API const char* rlk_backend_id(void) { return kBackendId; }

RLK_API uint64_t rlk_call_count(int which) {
  if (which < 0 || which > 7) return 0;
  return g_calls[which].load(std::memory_order_relaxed);
}

RLK_API int rlk_abi_version(void) { return kAbiVersion; }

RLK_API rlk_status rlk_profile_begin(void) {
  std::lock_guard<std::mutex> lk(g_prof.mu);
  g_prof.recs.clear();
  g_prof.next = 0;
  g_prof.failed = false;
  g_prof.on.store(true);
  return RLK_OK;
}

RLK_API rlk_status rlk_profile_end(double* total_ms, uint64_t* launches, int n) {
  if (n < 0 || (n > 0 && (!total_ms || !launches))) return RLK_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(g_prof.mu);
  g_prof.on.store(false);
  for (int i = 0; i < n; ++i) {
    total_ms[i] = 0.0;
    launches[i] = 0;
  }
  rlk_status st = g_prof.failed ? RLK_ERR_HIP : RLK_OK;
  for (const auto& r : g_prof.recs) {
    if (!r.b) continue;
    if (hipEventSynchronize(r.b) != hipSuccess) {
      st = RLK_ERR_HIP;
      continue;
    }
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) {
      st = RLK_ERR_HIP;
      continue;
    }
    if (r.id >= 0 && r.id < n) {
      total_ms[r.id] += ms;
      launches[r.id] += 1;
    }
  }
  g_prof.recs.clear();
  g_prof.next = 0;
  return st;
}

RLK_API int rlk_profile_kernel_count(void) { return rlk::K_COUNT; }

RLK_API const char* rlk_profile_kernel_name(int id) {
  return (id >= 0 && id < rlk::K_COUNT) ? rlk::kKernelNames[id] : "";
}

}  // extern "C"
