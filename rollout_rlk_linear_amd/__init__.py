"""Python binding of the gfx950 fused, batch-invariant linear log-prob.

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``librlk_linear.so`` behind the C ABI declared in
``include/rlk_linear.h``. PyTorch supplies device memory and the stream.
There is no fallback: if the library is missing or the device is not gfx950,
calls raise.

    logp, entropy = linear_logp(hidden, weight, targets)           # autograd-aware
    out = fwd(hidden, weight, targets)                              # dict: logp, entropy, stats
    dH, dW = bwd(hidden, weight, targets, out["stats"], dlogp)      # gradients
    parts = fwd(hidden, W_slice, targets, vocab_start=a, vocab_total=V)["stats"]
    logp, entropy, stats = combine_host([parts_0, parts_1, ...])    # fixed-order merge
    pw = pack_weight(W); out = fwd_packed(hidden, pw, targets)       # rollout: same bits as fwd

The operator is the linear-logp provider of the pages on RL-Kernel (page
"VIME Qwen3-8B TP4/CP2 200-round consistency experiment", section
"User-facing operator matrix": it stands in for VIME's
calculate_log_probs_and_entropy): logp of the target token and entropy of the
softmax of hidden @ W^T, with every row bitwise independent of the batch.
"""

from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "librlk_linear.so")

RLK_OK = 0
RLK_DH_F32 = 1
STATUS_NAMES = {0: "RLK_OK", 1: "RLK_ERR_INVALID_ARG", 2: "RLK_ERR_UNSUPPORTED_SHAPE",
                3: "RLK_ERR_WORKSPACE_TOO_SMALL", 4: "RLK_ERR_UNSUPPORTED_DEVICE",
                5: "RLK_ERR_HIP", 6: "RLK_ERR_SCRATCH_LIMIT"}

_lib = None


class RlkError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


def load_library(path: str | None = None):
    """Load librlk_linear.so (built in-tree by ``_build.py``); raise if absent."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m rollout_rlk_linear_amd._build` "
                           "(there is no non-HIP fallback)")
    lib = ctypes.CDLL(p)
    vp, i64, sz, f32p, i32p, u32 = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t,
                                    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint32)
    lib.rlk_linear_logp_fwd_workspace_bytes.argtypes = [i64, i64, i64]
    lib.rlk_linear_logp_fwd_workspace_bytes.restype = sz
    lib.rlk_linear_logp_bwd_workspace_bytes.argtypes = [i64, i64, i64, u32, ctypes.c_int]
    lib.rlk_linear_logp_bwd_workspace_bytes.restype = sz
    lib.rlk_linear_logp_fwd.argtypes = [vp, vp, i32p, i64, i64, i64, i64, i64, f32p, f32p, f32p,
                                        vp, sz, vp]
    lib.rlk_linear_logp_fwd.restype = ctypes.c_int
    lib.rlk_linear_logp_fwd_noalloc.argtypes = [vp, vp, i32p, i64, i64, i64, i64, i64, f32p, f32p,
                                                f32p, vp]
    lib.rlk_linear_logp_fwd_noalloc.restype = ctypes.c_int
    lib.rlk_linear_logp_fwd_packed_workspace_bytes.argtypes = [i64, i64, i64]
    lib.rlk_linear_logp_fwd_packed_workspace_bytes.restype = sz
    lib.rlk_linear_pack_weight_bytes.argtypes = [i64, i64, i64, i64]
    lib.rlk_linear_pack_weight_bytes.restype = sz
    lib.rlk_linear_pack_weight.argtypes = [vp, i64, i64, i64, i64, vp, sz, vp]
    lib.rlk_linear_pack_weight.restype = ctypes.c_int
    lib.rlk_linear_logp_fwd_packed.argtypes = [vp, vp, sz, i32p, i64, i64, i64, i64, i64, f32p,
                                               f32p, f32p, vp, sz, vp]
    lib.rlk_linear_logp_fwd_packed.restype = ctypes.c_int
    lib.rlk_linear_logp_bwd.argtypes = [vp, vp, i32p, i64, i64, i64, i64, i64, f32p, f32p, f32p,
                                        vp, f32p, u32, vp, sz, vp]
    lib.rlk_linear_logp_bwd.restype = ctypes.c_int
    lib.rlk_linear_logp_combine_host.argtypes = [f32p, i64, i64, f32p, f32p, f32p]
    lib.rlk_linear_logp_combine_host.restype = ctypes.c_int
    lib.rlk_linear_logp_combine.argtypes = [f32p, i64, i64, f32p, f32p, f32p, vp]
    lib.rlk_linear_logp_combine.restype = ctypes.c_int
    lib.rlk_linear_logp_dh_merge.argtypes = [f32p, i64, i64, i64, vp, u32, vp]
    lib.rlk_linear_logp_dh_merge.restype = ctypes.c_int
    lib.rlk_status_string.argtypes = [ctypes.c_int]
    lib.rlk_status_string.restype = ctypes.c_char_p
    lib.rlk_backend_id.argtypes = []
    lib.rlk_backend_id.restype = ctypes.c_char_p
    lib.rlk_call_count.argtypes = [ctypes.c_int]
    lib.rlk_call_count.restype = ctypes.c_uint64
    lib.rlk_abi_version.argtypes = []
    lib.rlk_abi_version.restype = ctypes.c_int
    lib.rlk_profile_begin.argtypes = []
    lib.rlk_profile_begin.restype = ctypes.c_int
    lib.rlk_profile_end.argtypes = [vp, vp, ctypes.c_int]
    lib.rlk_profile_end.restype = ctypes.c_int
    lib.rlk_profile_kernel_count.argtypes = []
    lib.rlk_profile_kernel_count.restype = ctypes.c_int
    lib.rlk_profile_kernel_name.argtypes = [ctypes.c_int]
    lib.rlk_profile_kernel_name.restype = ctypes.c_char_p
    lib.rlk_microbench_copy.argtypes = [vp, vp, sz, vp]
    lib.rlk_microbench_copy.restype = ctypes.c_int
    lib.rlk_lora_linear_workspace_bytes.argtypes = [i64, i64, i64, i64]
    lib.rlk_lora_linear_workspace_bytes.restype = sz
    lib.rlk_lora_linear_fwd.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_float, vp, vp,
                                        sz, vp]
    lib.rlk_lora_linear_fwd.restype = ctypes.c_int
    lib.rlk_lora_linear_bwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_float, vp,
                                        f32p, f32p, vp, sz, vp]
    lib.rlk_lora_linear_bwd.restype = ctypes.c_int
    lib.rlk_microbench_read.argtypes = [vp, sz, vp, i64, vp]
    lib.rlk_microbench_read.restype = ctypes.c_int
    lib.rlk_microbench_mfma.argtypes = [vp, i64, i64, vp]
    lib.rlk_microbench_mfma.restype = ctypes.c_int
    lib.rlk_microbench_mfma_clock.argtypes = [vp, i64, i64, ctypes.c_int, vp,
                                              ctypes.POINTER(ctypes.c_int64), vp]
    lib.rlk_microbench_mfma_clock.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def _check(status: int):
    if status != RLK_OK:
        lib = load_library()
        raise RlkError(status, lib.rlk_status_string(status).decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def backend_id() -> str:
    return load_library().rlk_backend_id().decode()


def call_count(which: int) -> int:
    return int(load_library().rlk_call_count(which))


def profile_begin():
    """Start the library's per-launch HIP-event timer."""
    _check(load_library().rlk_profile_begin())


def profile_end() -> dict:
    """Stop the timer; returns {kernel name: (summed ms, launches)}."""
    lib = load_library()
    n = lib.rlk_profile_kernel_count()
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_uint64 * n)()
    _check(lib.rlk_profile_end(ctypes.cast(ms, ctypes.c_void_p), ctypes.cast(cnt, ctypes.c_void_p), n))
    return {lib.rlk_profile_kernel_name(i).decode(): (float(ms[i]), int(cnt[i])) for i in range(n)}


def microbench_copy(dst: torch.Tensor, src: torch.Tensor):
    """Enqueue one copy of src's bytes into dst (``rlk_microbench_copy``)."""
    if dst.nbytes != src.nbytes or not (dst.is_cuda and src.is_cuda and dst.is_contiguous()
                                        and src.is_contiguous()):
        raise ValueError("dst and src must be contiguous device tensors of equal size")
    _check(load_library().rlk_microbench_copy(_ptr(dst), _ptr(src), src.nbytes, _stream(src.device)))


def microbench_read(src: torch.Tensor, sink: torch.Tensor, workgroups: int):
    """Linear LDS-DMA read of src (a multiple of 8 KB); see rlk_microbench.h."""
    _check(load_library().rlk_microbench_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink),
                                              workgroups, _stream(src.device)))


def microbench_mfma(sink: torch.Tensor, workgroups: int, iters: int) -> float:
    """Enqueue the MFMA-rate kernel; returns the flops it performs."""
    if not (sink.is_cuda and sink.dtype == torch.float32 and sink.numel() >= 4):
        raise ValueError("sink must be a device fp32 tensor of at least 4 elements")
    _check(load_library().rlk_microbench_mfma(_ptr(sink), workgroups, iters, _stream(sink.device)))
    return float(workgroups) * 4 * iters * 32 * 16384


def microbench_mfma_clock(sink: torch.Tensor, clocks: torch.Tensor, workgroups: int, iters: int,
                          shape: int):
    """Enqueue the clocked MFMA-rate kernel (shape 0: 16x16x32, 1: 32x32x16);
    clocks: device int64 [2 * workgroups]. Returns (flops, wall-clock kHz)."""
    if not (clocks.is_cuda and clocks.dtype == torch.int64 and clocks.numel() >= 2 * workgroups):
        raise ValueError("clocks must be a device int64 tensor of 2 * workgroups entries")
    khz = ctypes.c_int64(0)
    _check(load_library().rlk_microbench_mfma_clock(_ptr(sink), workgroups, iters, shape,
                                                    _ptr(clocks), ctypes.byref(khz),
                                                    _stream(sink.device)))
    return float(workgroups) * 4 * iters * 32 * 16384, int(khz.value)


def fwd_workspace_bytes(T: int, H: int, V: int) -> int:
    return int(load_library().rlk_linear_logp_fwd_workspace_bytes(T, H, V))


def bwd_workspace_bytes(T: int, H: int, V: int, flags: int = 0, want_dhidden: bool = True) -> int:
    return int(load_library().rlk_linear_logp_bwd_workspace_bytes(T, H, V, flags, int(want_dhidden)))


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def _reuse(out: dict, key: str, shape, dtype):
    """A caller-provided output tensor from ``out`` if it fits, else None."""
    t = out.get(key)
    if t is None or tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous():
        return None
    return t


def _check_inputs(hidden, weight, targets):
    if hidden.dtype != torch.bfloat16 or weight.dtype != torch.bfloat16:
        raise TypeError("hidden and weight must be bfloat16")
    if targets.dtype != torch.int32:
        raise TypeError("targets must be int32")
    for name, t in (("hidden", hidden), ("weight", weight), ("targets", targets)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")


def _outputs(out: dict, T: int, full: bool, want_logp: bool, want_entropy: bool,
             want_stats: bool, dev):
    logp = _reuse(out, "logp", (T,), torch.float32) if full and want_logp else None
    ent = _reuse(out, "entropy", (T,), torch.float32) if full and want_entropy else None
    stats = _reuse(out, "stats", (T, 4), torch.float32) if want_stats or not full else None
    if full and want_logp and logp is None:
        logp = torch.empty(T, dtype=torch.float32, device=dev)
    if full and want_entropy and ent is None:
        ent = torch.empty(T, dtype=torch.float32, device=dev)
    if (want_stats or not full) and stats is None:
        stats = torch.empty(T, 4, dtype=torch.float32, device=dev)
    return logp, ent, stats


def _fwd_workspace(out: dict, key: str, nws: int, dev) -> torch.Tensor:
    ws = out.get(key)
    if ws is None or ws.numel() < nws:
        ws = _workspace(nws, dev)
    out[key] = ws
    return ws


def fwd(hidden: torch.Tensor, weight: torch.Tensor, targets: torch.Tensor, *,
        vocab_start: int = 0, vocab_total: int | None = None, want_logp: bool = True,
        want_entropy: bool = True, want_stats: bool = True, out: dict | None = None):
    """Forward through ``rlk_linear_logp_fwd``. Returns dict(logp, entropy, stats).

    For a vocabulary slice (``vocab_start``/``vocab_total``) only ``stats`` is
    produced: the slice's (m, R, B, zy) record per row, fp32 [T, 4].
    """
    lib = load_library()
    _check_inputs(hidden, weight, targets)
    T, H = hidden.shape
    V = weight.shape[0]
    vt = V if vocab_total is None else vocab_total
    full = vocab_start == 0 and V == vt
    dev = hidden.device
    out = {} if out is None else out
    logp, ent, stats = _outputs(out, T, full, want_logp, want_entropy, want_stats, dev)
    ws = _fwd_workspace(out, "_ws_fwd", lib.rlk_linear_logp_fwd_workspace_bytes(T, H, V), dev)
    out.update({"logp": logp, "entropy": ent, "stats": stats})
    _check(lib.rlk_linear_logp_fwd(_ptr(hidden), _ptr(weight), _ptr(targets), T, H, V,
                                   vocab_start, vt, _ptr(logp), _ptr(ent), _ptr(stats),
                                   _ptr(ws), ws.numel(), _stream(dev)))
    return {"logp": logp, "entropy": ent, "stats": stats}


def fwd_noalloc(hidden: torch.Tensor, weight: torch.Tensor, targets: torch.Tensor, *,
                vocab_start: int = 0, vocab_total: int | None = None, want_logp: bool = True,
                want_entropy: bool = True, want_stats: bool = True, out: dict | None = None):
    """Forward through ``rlk_linear_logp_fwd_noalloc``: the library's static
    scratch instead of a workspace (same bits as ``fwd``). Outputs come from
    ``out`` when they fit, else are allocated here (the library allocates
    nothing). Raises RlkError(RLK_ERR_SCRATCH_LIMIT) when the records of
    (T, H, V) exceed the scratch."""
    lib = load_library()
    _check_inputs(hidden, weight, targets)
    T, H = hidden.shape
    V = weight.shape[0]
    vt = V if vocab_total is None else vocab_total
    full = vocab_start == 0 and V == vt
    dev = hidden.device
    out = {} if out is None else out
    logp, ent, stats = _outputs(out, T, full, want_logp, want_entropy, want_stats, dev)
    out.update({"logp": logp, "entropy": ent, "stats": stats})
    _check(lib.rlk_linear_logp_fwd_noalloc(_ptr(hidden), _ptr(weight), _ptr(targets), T, H, V,
                                           vocab_start, vt, _ptr(logp), _ptr(ent), _ptr(stats),
                                           _stream(dev)))
    return {"logp": logp, "entropy": ent, "stats": stats}


class PackedWeight:
    """W rearranged by ``rlk_linear_pack_weight`` for (H, V, vocab_start, vocab_total)."""

    def __init__(self, data: torch.Tensor, H: int, V: int, vocab_start: int, vocab_total: int):
        self.data, self.H, self.V = data, H, V
        self.vocab_start, self.vocab_total = vocab_start, vocab_total


def pack_weight_bytes(H: int, V: int, vocab_start: int = 0, vocab_total: int | None = None) -> int:
    vt = V if vocab_total is None else vocab_total
    return int(load_library().rlk_linear_pack_weight_bytes(H, V, vocab_start, vt))


def pack_weight(weight: torch.Tensor, *, vocab_start: int = 0, vocab_total: int | None = None,
                out: PackedWeight | None = None) -> PackedWeight:
    """Packed copy of ``weight`` for ``fwd_packed`` (same slicing arguments)."""
    lib = load_library()
    if weight.dtype != torch.bfloat16 or not weight.is_cuda or not weight.is_contiguous():
        raise ValueError("weight must be a contiguous bfloat16 device tensor")
    V, H = weight.shape
    vt = V if vocab_total is None else vocab_total
    nbytes = lib.rlk_linear_pack_weight_bytes(H, V, vocab_start, vt)
    if nbytes == 0:
        raise RlkError(1, "pack_weight: unsupported shape or slicing")
    data = out.data if out is not None and out.data.numel() >= nbytes else None
    if data is None:
        data = torch.empty(nbytes, dtype=torch.uint8, device=weight.device)
    _check(lib.rlk_linear_pack_weight(_ptr(weight), H, V, vocab_start, vt, _ptr(data), data.numel(),
                                      _stream(weight.device)))
    return PackedWeight(data, H, V, vocab_start, vt)


def fwd_packed(hidden: torch.Tensor, packed: PackedWeight, targets: torch.Tensor, *,
               want_logp: bool = True, want_entropy: bool = True, want_stats: bool = True,
               out: dict | None = None):
    """Forward through ``rlk_linear_logp_fwd_packed``: same results, bit for bit, as
    ``fwd`` over the weight ``packed`` was made from."""
    lib = load_library()
    if hidden.dtype != torch.bfloat16 or targets.dtype != torch.int32:
        raise TypeError("hidden must be bfloat16 and targets int32")
    for name, t in (("hidden", hidden), ("targets", targets)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    T, H = hidden.shape
    if H != packed.H:
        raise ValueError(f"hidden has H={H}, the packed weight H={packed.H}")
    V, vs0, vt = packed.V, packed.vocab_start, packed.vocab_total
    full = vs0 == 0 and V == vt
    dev = hidden.device
    out = {} if out is None else out
    logp, ent, stats = _outputs(out, T, full, want_logp, want_entropy, want_stats, dev)
    ws = _fwd_workspace(out, "_ws_fwdp", lib.rlk_linear_logp_fwd_packed_workspace_bytes(T, H, V), dev)
    out.update({"logp": logp, "entropy": ent, "stats": stats})
    _check(lib.rlk_linear_logp_fwd_packed(_ptr(hidden), _ptr(packed.data), packed.data.numel(),
                                          _ptr(targets), T, H, V, vs0, vt, _ptr(logp), _ptr(ent),
                                          _ptr(stats), _ptr(ws), ws.numel(), _stream(dev)))
    return {"logp": logp, "entropy": ent, "stats": stats}


def bwd(hidden: torch.Tensor, weight: torch.Tensor, targets: torch.Tensor, stats: torch.Tensor,
        dlogp: torch.Tensor | None, dentropy: torch.Tensor | None = None, *,
        vocab_start: int = 0, vocab_total: int | None = None, want_dhidden: bool = True,
        want_dweight: bool = True, dhidden_f32: bool = False, out: dict | None = None):
    """Backward through ``rlk_linear_logp_bwd``. Returns (dhidden, dweight).

    ``stats`` is the whole-vocabulary record (fwd's ``stats`` or the combined
    one for slices). dhidden is bf16 [T,H] (fp32 with ``dhidden_f32``),
    dweight fp32 [V,H].
    """
    lib = load_library()
    _check_inputs(hidden, weight, targets)
    T, H = hidden.shape
    V = weight.shape[0]
    vt = V if vocab_total is None else vocab_total
    dev = hidden.device
    out = {} if out is None else out
    for name, t in (("stats", stats), ("dlogp", dlogp), ("dentropy", dentropy)):
        if t is not None and (t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous fp32 device tensor")
    flags = RLK_DH_F32 if dhidden_f32 else 0
    dh = (_reuse(out, "dhidden", (T, H), torch.float32 if dhidden_f32 else torch.bfloat16)
          if want_dhidden else None)
    dw = _reuse(out, "dweight", (V, H), torch.float32) if want_dweight else None
    if want_dhidden and dh is None:
        dh = torch.empty(T, H, dtype=torch.float32 if dhidden_f32 else torch.bfloat16, device=dev)
    if want_dweight and dw is None:
        dw = torch.empty(V, H, dtype=torch.float32, device=dev)
    nws = lib.rlk_linear_logp_bwd_workspace_bytes(T, H, V, flags, int(want_dhidden))
    ws = out.get("_ws_bwd")
    if ws is None or ws.numel() < nws:
        ws = _workspace(nws, dev)
    out.update({"dhidden": dh, "dweight": dw, "_ws_bwd": ws})
    _check(lib.rlk_linear_logp_bwd(_ptr(hidden), _ptr(weight), _ptr(targets), T, H, V,
                                   vocab_start, vt, _ptr(stats), _ptr(dlogp), _ptr(dentropy),
                                   _ptr(dh), _ptr(dw), flags, _ptr(ws), ws.numel(), _stream(dev)))
    return dh, dw


def combine_host(partials):
    """Merge per-slice stats (list of [T,4] fp32, CPU or device, slices in
    vocabulary order) by the library's fixed merge tree.

    Runs ``rlk_linear_logp_combine_host`` on the CPU. Returns (logp, entropy,
    stats) as CPU fp32 tensors.
    """
    lib = load_library()
    parts = torch.stack([p.detach().to("cpu", torch.float32) for p in partials]).contiguous()
    S, T = parts.shape[0], parts.shape[1]
    logp = torch.empty(T, dtype=torch.float32)
    ent = torch.empty(T, dtype=torch.float32)
    stats = torch.empty(T, 4, dtype=torch.float32)
    _check(lib.rlk_linear_logp_combine_host(_ptr(parts), S, T, _ptr(logp), _ptr(ent), _ptr(stats)))
    return logp, ent, stats


def combine(partials, out: dict | None = None):
    """Merge per-slice stats on the device (``rlk_linear_logp_combine``).

    ``partials``: list of [T,4] fp32 device tensors, or one [S,T,4] tensor,
    slices in vocabulary order. Returns dict(logp, entropy, stats) on the
    same device; the bits equal those of a forward call covering the same
    aligned virtual slices.
    """
    lib = load_library()
    parts = partials if isinstance(partials, torch.Tensor) else torch.stack(list(partials))
    parts = parts.contiguous()
    if parts.dim() != 3 or parts.shape[2] != 4 or parts.dtype != torch.float32 or not parts.is_cuda:
        raise ValueError("partials must be device fp32 [S,T,4] (or a list of [T,4])")
    S, T = parts.shape[0], parts.shape[1]
    out = {} if out is None else out
    logp = _reuse(out, "logp", (T,), torch.float32)
    ent = _reuse(out, "entropy", (T,), torch.float32)
    stats = _reuse(out, "stats", (T, 4), torch.float32)
    if logp is None:
        logp = torch.empty(T, dtype=torch.float32, device=parts.device)
    if ent is None:
        ent = torch.empty(T, dtype=torch.float32, device=parts.device)
    if stats is None:
        stats = torch.empty(T, 4, dtype=torch.float32, device=parts.device)
    out.update({"logp": logp, "entropy": ent, "stats": stats})
    _check(lib.rlk_linear_logp_combine(_ptr(parts), S, T, _ptr(logp), _ptr(ent), _ptr(stats),
                                       _stream(parts.device)))
    return {"logp": logp, "entropy": ent, "stats": stats}


def dh_merge(parts, f32: bool = False, out: torch.Tensor | None = None) -> torch.Tensor:
    """Sum fp32 dH contributions of slice calls (``bwd(..., dhidden_f32=True)`` of
    each slice, in vocabulary order) by the library's fixed tree
    (``rlk_linear_logp_dh_merge``); bf16 [T,H] (fp32 with ``f32``)."""
    lib = load_library()
    p = parts if isinstance(parts, torch.Tensor) else torch.stack(list(parts))
    p = p.contiguous()
    if p.dim() != 3 or p.dtype != torch.float32 or not p.is_cuda:
        raise ValueError("parts must be device fp32 [S,T,H] (or a list of [T,H])")
    S, T, H = p.shape
    dt = torch.float32 if f32 else torch.bfloat16
    if out is None or tuple(out.shape) != (T, H) or out.dtype != dt or not out.is_contiguous():
        out = torch.empty(T, H, dtype=dt, device=p.device)
    _check(lib.rlk_linear_logp_dh_merge(_ptr(p), S, T, H, _ptr(out), RLK_DH_F32 if f32 else 0,
                                        _stream(p.device)))
    return out


class LinearLogp(torch.autograd.Function):
    """Autograd wrapper: forward (logp, entropy); backward (dhidden, dweight)."""

    @staticmethod
    def forward(ctx, hidden, weight, targets):
        o = fwd(hidden, weight, targets)
        ctx.save_for_backward(hidden, weight, targets, o["stats"])
        ctx.mark_non_differentiable(o["stats"])
        return o["logp"], o["entropy"]

    @staticmethod
    def backward(ctx, dlogp, dentropy):
        hidden, weight, targets, stats = ctx.saved_tensors
        dl = None if dlogp is None else dlogp.float().contiguous()
        de = None if dentropy is None else dentropy.float().contiguous()
        dh, dw = bwd(hidden, weight, targets, stats, dl, de,
                     want_dhidden=ctx.needs_input_grad[0], want_dweight=ctx.needs_input_grad[1])
        return dh, (None if dw is None else dw.to(weight.dtype)), None


def linear_logp(hidden, weight, targets):
    """(logp, entropy) per token; differentiable in hidden and weight."""
    return LinearLogp.apply(hidden, weight, targets)


# ------------------------------------------------------------ LoRA linear ----

def _lora_check(x, W, A, B):
    for name, t in (("x", x), ("W", W), ("A", A), ("B", B)):
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bfloat16 device tensor")
    T, K = x.shape
    N = W.shape[0]
    r = A.shape[0]
    if W.shape != (N, K) or A.shape != (r, K) or B.shape != (N, r):
        raise ValueError(f"shapes x{tuple(x.shape)} W{tuple(W.shape)} A{tuple(A.shape)} "
                         f"B{tuple(B.shape)} do not form x[T,K] W[N,K] A[r,K] B[N,r]")
    return T, K, N, r


def lora_fwd(x, W, A, B, scale: float = 1.0, out: torch.Tensor | None = None, ws=None):
    """y = x W^T + scale (x A^T) B^T through ``rlk_lora_linear_fwd`` (bf16 [T,N])."""
    lib = load_library()
    T, K, N, r = _lora_check(x, W, A, B)
    if out is not None:
        _lora_out(out, (T, N), torch.bfloat16, x.device, "out")
    y = out if out is not None else torch.empty(T, N, dtype=torch.bfloat16, device=x.device)
    nws = lib.rlk_lora_linear_workspace_bytes(T, K, N, r)
    ws = ws if ws is not None and ws.numel() >= nws else _workspace(nws, x.device)
    _check(lib.rlk_lora_linear_fwd(_ptr(x), _ptr(W), _ptr(A), _ptr(B), T, K, N, r, float(scale),
                                   _ptr(y), _ptr(ws), ws.numel(), _stream(x.device)))
    return y


def _lora_out(t, shape, dtype, device, what):
    if (not isinstance(t, torch.Tensor) or t.dtype != dtype or t.device != device
            or not t.is_contiguous() or tuple(t.shape) != tuple(shape)):
        raise ValueError(f"{what} must be a contiguous {dtype} tensor {list(shape)} on {device}")


def lora_bwd(x, W, A, B, dy, scale: float = 1.0, *, want_dx=True, want_da=True, want_db=True,
             ws=None, out=None):
    """(dx bf16 [T,K], dA fp32 [r,K], dB fp32 [N,r]) through ``rlk_lora_linear_bwd``;
    None where not wanted. W is frozen: no gradient. ``out``: optional
    (dx, dA, dB) tensors of those shapes to write into (each of them used only
    where wanted)."""
    lib = load_library()
    T, K, N, r = _lora_check(x, W, A, B)
    if dy.dtype != torch.bfloat16 or not dy.is_cuda or not dy.is_contiguous() or dy.shape != (T, N):
        raise ValueError("dy must be a contiguous bfloat16 device tensor [T, N]")
    dev = x.device
    if out is not None:
        odx, oda, odb = out
        _lora_out(odx, (T, K), torch.bfloat16, dev, "out dx")
        _lora_out(oda, (r, K), torch.float32, dev, "out dA")
        _lora_out(odb, (N, r), torch.float32, dev, "out dB")
    dx = (odx if out is not None else torch.empty(T, K, dtype=torch.bfloat16, device=dev)) \
        if want_dx else None
    da = (oda if out is not None else torch.empty(r, K, dtype=torch.float32, device=dev)) \
        if want_da else None
    db = (odb if out is not None else torch.empty(N, r, dtype=torch.float32, device=dev)) \
        if want_db else None
    nws = lib.rlk_lora_linear_workspace_bytes(T, K, N, r)
    ws = ws if ws is not None and ws.numel() >= nws else _workspace(nws, dev)
    _check(lib.rlk_lora_linear_bwd(_ptr(x), _ptr(W), _ptr(A), _ptr(B), _ptr(dy), T, K, N, r,
                                   float(scale), _ptr(dx), _ptr(da), _ptr(db), _ptr(ws), ws.numel(),
                                   _stream(dev)))
    return dx, da, db


class _LoraLinearFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, W, A, B, scale):
        ctx.save_for_backward(x, W, A, B)
        ctx.scale = scale
        return lora_fwd(x, W, A, B, scale)

    @staticmethod
    def backward(ctx, dy):
        x, W, A, B = ctx.saved_tensors
        dx, da, db = lora_bwd(x, W, A, B, dy.contiguous(), ctx.scale,
                              want_dx=ctx.needs_input_grad[0], want_da=ctx.needs_input_grad[2],
                              want_db=ctx.needs_input_grad[3])
        return (dx, None, None if da is None else da.to(A.dtype),
                None if db is None else db.to(B.dtype), None)


def lora_linear(x, W, A, B, scale: float = 1.0):
    """Autograd-aware LoRA linear (W frozen: it never receives a gradient)."""
    return _LoraLinearFn.apply(x, W, A, B, scale)

