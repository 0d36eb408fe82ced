"""The C-ABI library on the host (no GPU needed).

* it loads and exports every symbol that include/rlk_linear.h declares;
* every argument error is returned as its status code before any HIP call
  (fake device pointers are never dereferenced on the host);
* workspace queries follow the documented sizes;
* the host-side slice combine agrees with the float64 oracle.
"""

import ctypes
import glob
import math
import os
import re

import numpy as np
import pytest
import torch

import rollout_rlk_linear_amd as rlk
from oracle import finalize_partials, forward_f64, merge_partials, slice_partials_f64

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))

OK, INVALID, SHAPE, WS_SMALL, DEVICE, HIPERR, SCRATCH = 0, 1, 2, 3, 4, 5, 6
P = ctypes.c_void_p(1 << 20)  # aligned fake device pointer, never dereferenced on the host
NULL = None


def declared_symbols():
    names = []
    for h in HEADERS:
        names += re.findall(r"RLK_API\s+[\w\s\*]+?\b(rlk_\w+)\s*\(", open(h).read())
    return names


def test_header_declares_the_entry_points():
    names = declared_symbols()
    for n in ["rlk_linear_logp_fwd", "rlk_linear_logp_bwd", "rlk_linear_logp_fwd_workspace_bytes",
              "rlk_linear_logp_bwd_workspace_bytes", "rlk_linear_logp_combine_host",
              "rlk_status_string", "rlk_backend_id", "rlk_call_count", "rlk_abi_version",
              "rlk_microbench_copy", "rlk_microbench_mfma"]:
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(rlk.LIB_PATH)
    for n in declared_symbols():
        assert hasattr(raw, n), n


def test_combine_argument_errors(lib):
    raw = ctypes.CDLL(rlk.LIB_PATH)
    raw.rlk_linear_logp_combine.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_void_p]
    c = raw.rlk_linear_logp_combine
    assert c(P, 0, 4, P, P, P, NULL) == INVALID                    # no slices
    assert c(P, 1025, 4, P, P, P, NULL) == INVALID                 # too many slices
    assert c(P, 4, -1, P, P, P, NULL) == INVALID
    assert c(P, 4, 4, NULL, NULL, NULL, NULL) == INVALID           # nothing requested
    assert c(NULL, 4, 4, P, P, P, NULL) == INVALID
    assert c(ctypes.c_void_p((1 << 20) + 4), 4, 4, P, P, P, NULL) == INVALID  # misaligned
    assert c(P, 4, 4, P, P, ctypes.c_void_p((1 << 20) + 4), NULL) == INVALID
    assert c(P, 4, 0, P, P, P, NULL) == OK                         # T == 0: no-op
    assert lib.rlk_call_count(3) >= 1


def test_combine_host_tree_order():
    # three records whose merge order is visible in fp32: the tree merges
    # (r0 + r1) first and then r2, which equals a left fold for S = 3 but
    # not for S = 4 where (r0 + r1) + (r2 + r3) is the defined order
    raw = ctypes.CDLL(rlk.LIB_PATH)
    raw.rlk_linear_logp_combine_host.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                                 ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    r = np.random.default_rng(11)
    S, T = 4, 512
    parts = np.zeros((S, T, 4), dtype=np.float32)
    parts[..., 0] = r.normal(0, 3, (S, T))
    parts[..., 1] = r.uniform(0, 50, (S, T))
    parts[..., 2] = -r.uniform(0, 80, (S, T))
    parts[..., 3] = -np.inf
    out = np.zeros((T, 4), dtype=np.float32)
    raw.rlk_linear_logp_combine_host(parts.ctypes.data, S, T, None, None, out.ctypes.data)

    def merge(a, b):
        base_left = not (b[0] > a[0])
        bb, oo = (a, b) if base_left else (b, a)
        if oo[0] == -np.inf:
            return bb.copy()
        d = np.float32(oo[0] - bb[0])
        e = np.float32(np.exp(np.float64(d)))
        one_r = np.float32(1) + oo[1]
        return np.array([bb[0], bb[1] + e * one_r, bb[2] + e * (oo[2] + one_r * d), -np.inf],
                        dtype=np.float32)

    for t in range(0, T, 37):
        want = merge(merge(parts[0, t], parts[1, t]), merge(parts[2, t], parts[3, t]))
        np.testing.assert_allclose(out[t, :3], want[:3], rtol=2e-6)


def test_microbench_argument_errors():
    raw = ctypes.CDLL(rlk.LIB_PATH)
    raw.rlk_microbench_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    raw.rlk_microbench_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
    Q = ctypes.c_void_p(1 << 21)
    assert raw.rlk_microbench_copy(NULL, Q, 1024, NULL) == INVALID
    assert raw.rlk_microbench_copy(P, Q, 1000, NULL) == INVALID             # not a multiple of 16
    assert raw.rlk_microbench_copy(ctypes.c_void_p((1 << 20) + 8), Q, 1024, NULL) == INVALID
    assert raw.rlk_microbench_copy(P, Q, 0, NULL) == INVALID
    assert raw.rlk_microbench_mfma(NULL, 256, 10, NULL) == INVALID
    assert raw.rlk_microbench_mfma(P, 0, 10, NULL) == INVALID
    assert raw.rlk_microbench_mfma(P, 256, 0, NULL) == INVALID
    assert raw.rlk_microbench_mfma(P, 256, (1 << 24) + 1, NULL) == INVALID
    raw.rlk_microbench_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                        ctypes.c_int64, ctypes.c_void_p]
    assert raw.rlk_microbench_read(NULL, 8192, P, 256, NULL) == INVALID
    assert raw.rlk_microbench_read(Q, 8192 + 16, P, 256, NULL) == INVALID   # not whole 8 KB stages
    assert raw.rlk_microbench_read(Q, 8192, NULL, 256, NULL) == INVALID
    assert raw.rlk_microbench_read(Q, 8192, P, 0, NULL) == INVALID
    assert raw.rlk_microbench_read(ctypes.c_void_p((1 << 21) + 8), 8192, P, 256, NULL) == INVALID
    raw.rlk_microbench_mfma_clock.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                              ctypes.c_int, ctypes.c_void_p,
                                              ctypes.POINTER(ctypes.c_int64), ctypes.c_void_p]
    khz = ctypes.c_int64(0)
    mc = raw.rlk_microbench_mfma_clock
    assert mc(NULL, 256, 10, 0, Q, ctypes.byref(khz), NULL) == INVALID
    assert mc(P, 256, 10, 2, Q, ctypes.byref(khz), NULL) == INVALID        # unknown shape
    assert mc(P, 256, 10, 1, NULL, ctypes.byref(khz), NULL) == INVALID     # no clock buffer
    assert mc(P, 256, 10, 1, Q, None, NULL) == INVALID                     # no rate output
    assert mc(P, 0, 10, 0, Q, ctypes.byref(khz), NULL) == INVALID
    assert mc(P, 256, 0, 0, Q, ctypes.byref(khz), NULL) == INVALID


def test_provenance(lib):
    assert lib.rlk_backend_id().decode() == "rlk.linear_logp.bitwise.gfx950.v1"
    assert lib.rlk_abi_version() == 1
    for s in range(7):
        assert lib.rlk_status_string(s)
    assert b"scratch" in lib.rlk_status_string(SCRATCH)
    assert lib.rlk_status_string(99).decode() == "unknown status"
    assert lib.rlk_call_count(7) == 0


def fwd(lib, hidden=P, weight=P, targets=P, T=4, H=64, V=100, vs=0, vt=None, logp=P, ent=P,
        stats=P, ws=P, nws=1 << 30):
    vt = V if vt is None else vt
    return lib.rlk_linear_logp_fwd(hidden, weight, targets, T, H, V, vs, vt, logp, ent, stats, ws,
                                   nws, NULL)


def bwd(lib, hidden=P, weight=P, targets=P, T=4, H=64, V=100, vs=0, vt=None, stats=P, dl=P,
        de=NULL, dh=P, dw=P, flags=0, ws=P, nws=1 << 34):
    vt = V if vt is None else vt
    return lib.rlk_linear_logp_bwd(hidden, weight, targets, T, H, V, vs, vt, stats, dl, de, dh, dw,
                                   flags, ws, nws, NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(T=-1), INVALID), (dict(H=0), INVALID), (dict(V=0), INVALID),
    (dict(H=96), SHAPE), (dict(H=65536 + 64), SHAPE), (dict(T=(1 << 21) + 1), SHAPE),
    (dict(V=(1 << 24) + 1, vt=(1 << 24) + 1), SHAPE),
    (dict(vs=-1), INVALID), (dict(vt=50), INVALID), (dict(vs=10, vt=105), INVALID),
    (dict(vt=(1 << 31)), INVALID),
    (dict(vs=5, vt=200, stats=P), INVALID),              # slice with logp/entropy requested
    (dict(logp=NULL, ent=NULL, stats=NULL), INVALID),    # nothing requested
    (dict(weight=NULL), INVALID), (dict(hidden=NULL), INVALID), (dict(targets=NULL), INVALID),
    (dict(hidden=ctypes.c_void_p((1 << 20) + 2)), INVALID),   # misaligned
    (dict(stats=ctypes.c_void_p((1 << 20) + 4)), INVALID),
    (dict(nws=0), WS_SMALL), (dict(ws=NULL), INVALID),
])
def test_fwd_argument_errors(lib, kw, code):
    assert fwd(lib, **kw) == code


def test_fwd_slice_without_logp_passes_checks(lib):
    # a valid slice call gets past every argument check to the device check
    st = fwd(lib, vs=5, vt=200, logp=NULL, ent=NULL)
    assert st in (HIPERR, DEVICE) if not torch.cuda.is_available() else True


def test_fwd_T0_is_noop(lib):
    before = lib.rlk_call_count(0)
    assert fwd(lib, T=0, hidden=NULL, targets=NULL, ws=NULL, nws=0) == OK
    assert lib.rlk_call_count(0) == before + 1


@pytest.mark.parametrize("kw,code", [
    (dict(T=-1), INVALID), (dict(H=100), SHAPE), (dict(vs=1), INVALID),
    (dict(flags=2), INVALID), (dict(dh=NULL, dw=NULL), INVALID), (dict(stats=NULL), INVALID),
    (dict(hidden=NULL), INVALID), (dict(weight=NULL), INVALID),
    (dict(dh=ctypes.c_void_p((1 << 20) + 8)), INVALID),
    (dict(dw=ctypes.c_void_p((1 << 20) + 4)), INVALID),
    (dict(dl=ctypes.c_void_p((1 << 20) + 2)), INVALID),
    (dict(nws=1024), WS_SMALL), (dict(ws=ctypes.c_void_p((1 << 20) + 16)), INVALID),
])
def test_bwd_argument_errors(lib, kw, code):
    assert bwd(lib, **kw) == code


@pytest.mark.skipif(torch.cuda.is_available(), reason="host-only check of the no-device path")
def test_valid_call_without_device_reports_hip_error(lib):
    assert fwd(lib) in (HIPERR, DEVICE)
    assert bwd(lib) in (HIPERR, DEVICE)


def test_bwd_T0_without_dweight_is_noop(lib):
    assert bwd(lib, T=0, hidden=NULL, targets=NULL, stats=NULL, dw=NULL, ws=NULL, nws=0) == OK


def fwdp(lib, hidden=P, packed=P, npk=1 << 40, targets=P, T=4, H=64, V=100, vs=0, vt=None,
         logp=P, ent=P, stats=P, ws=P, nws=1 << 30):
    vt = V if vt is None else vt
    return lib.rlk_linear_logp_fwd_packed(hidden, packed, npk, targets, T, H, V, vs, vt, logp, ent,
                                          stats, ws, nws, NULL)


def test_pack_weight_bytes(lib):
    f = lib.rlk_linear_pack_weight_bytes
    # whole vocabulary 151936 = 4 virtual slices of 37984 rows = 297 units of 128 rows each
    assert f(4096, 151936, 0, 151936) == 4 * 297 * 128 * 4096 * 2
    # half of a 303872-row vocabulary: 2 slices of 75968 rows, 594 units each
    assert f(4096, 151936, 151936, 303872) == 2 * 594 * 128 * 4096 * 2
    # no virtual slicing (vocab_total not a multiple of 4): one slice of V rows
    assert f(64, 1001, 0, 1001) == 8 * 128 * 64 * 2
    assert f(96, 1000, 0, 1000) == 0        # H not a multiple of 64
    assert f(64, 0, 0, 1000) == 0
    assert f(64, 100, 950, 1000) == 0       # slice past the vocabulary


@pytest.mark.parametrize("kw,code", [
    (dict(weight=NULL), INVALID), (dict(packed=NULL), INVALID),
    (dict(packed=ctypes.c_void_p((1 << 20) + 8)), INVALID), (dict(H=96), SHAPE),
    (dict(npk=1000), WS_SMALL), (dict(vs=10, vt=105), INVALID),
])
def test_pack_weight_argument_errors(lib, kw, code):
    a = dict(weight=P, H=64, V=100, vs=0, vt=100, packed=P, npk=1 << 30)
    a.update(kw)
    assert lib.rlk_linear_pack_weight(a["weight"], a["H"], a["V"], a["vs"], a["vt"], a["packed"],
                                      a["npk"], NULL) == code


@pytest.mark.parametrize("kw,code", [
    (dict(npk=4 * 128 * 64 * 2 - 2), INVALID),   # (64, 100): 4 virtual slices, one unit each
    (dict(packed=NULL), INVALID), (dict(T=-1), INVALID), (dict(H=96), SHAPE),
    (dict(vs=5, vt=200, stats=P), INVALID), (dict(nws=0), WS_SMALL),
    (dict(hidden=ctypes.c_void_p((1 << 20) + 2)), INVALID),
])
def test_fwd_packed_argument_errors(lib, kw, code):
    assert fwdp(lib, **kw) == code


def test_fwd_packed_T0_is_noop(lib):
    before = lib.rlk_call_count(5)
    assert fwdp(lib, T=0, hidden=NULL, targets=NULL, ws=NULL, nws=0) == OK
    assert lib.rlk_call_count(5) == before + 1


def lora_fwd(lib, x=P, W=P, A=P, B=P, T=4, K=64, N=128, r=16, y=P, ws=P, nws=1 << 20):
    return lib.rlk_lora_linear_fwd(x, W, A, B, T, K, N, r, 1.0, y, ws, nws, NULL)


def lora_bwd(lib, x=P, W=P, A=P, B=P, dy=P, T=4, K=64, N=128, r=16, dx=P, da=P, db=P, ws=P,
             nws=1 << 20):
    return lib.rlk_lora_linear_bwd(x, W, A, B, dy, T, K, N, r, 1.0, dx, da, db, ws, nws, NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(T=-1), INVALID), (dict(K=0), INVALID), (dict(r=0), INVALID),
    (dict(K=96), SHAPE), (dict(N=100), SHAPE), (dict(r=65), SHAPE), (dict(K=65536 + 64), SHAPE),
    (dict(N=(1 << 20) + 64), SHAPE), (dict(T=(1 << 21) + 1), SHAPE),
    (dict(x=NULL), INVALID), (dict(W=NULL), INVALID), (dict(A=NULL), INVALID),
    (dict(B=NULL), INVALID), (dict(y=NULL), INVALID), (dict(ws=NULL), INVALID),
    (dict(x=ctypes.c_void_p((1 << 20) + 2)), INVALID), (dict(nws=4 * 16 * 8 - 1), WS_SMALL),
])
def test_lora_fwd_argument_errors(lib, kw, code):
    assert lora_fwd(lib, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(dx=NULL, da=NULL, db=NULL), INVALID), (dict(dy=NULL), INVALID), (dict(K=32), SHAPE),
    (dict(da=ctypes.c_void_p((1 << 20) + 4)), INVALID), (dict(nws=0), WS_SMALL),
])
def test_lora_bwd_argument_errors(lib, kw, code):
    assert lora_bwd(lib, **kw) == code


def test_lora_workspace_and_empty_forward(lib):
    f = lib.rlk_lora_linear_workspace_bytes
    # u and v: 2 x 33 x 16 fp32, rounded to 256; K = 5120 splits the forward's
    # contraction in 4: partials 4 x 33 x 5120 fp32
    assert f(33, 5120, 5120, 16) == 4352 + 4 * 33 * 5120 * 4
    assert f(33, 1024, 2048, 16) == 4352          # K, N < 2560: no split
    # dx's contraction over N = 8192 splits in 4: partials 4 x 33 x 1024 fp32
    assert f(33, 1024, 8192, 16) == 4352 + 4 * 33 * 1024 * 4
    assert f(0, 64, 64, 16) == 0 and f(4, 96, 64, 16) == 0
    assert lora_fwd(lib, T=0, x=NULL, y=NULL, ws=NULL, nws=0) == OK


@pytest.mark.parametrize("L", [64, 1216, 1280, 2496, 2560, 2624, 2688, 5056, 5120, 5184, 5248,
                               5376, 65536])
def test_lora_split_count_follows_the_length(lib, L):
    """The number of splits S of a contraction of length L is the largest of
    4 and 2 with L >= 1280 S and L a multiple of 64 S, else 1, and nothing
    else (not T, not the other dimension). S is read back from the size of
    the partials in the workspace (S x T x N fp32 for the forward's
    contraction over K, at N = 64 so that dx's over N is never split)."""
    expect = next((s for s in (4, 2) if L >= 1280 * s and L % (64 * s) == 0), 1)
    f = lib.rlk_lora_linear_workspace_bytes
    for T in (1, 33, 257):
        uv = (2 * T * 4 + 255) // 256 * 256           # u and v at r = 1
        part = (expect * T * 64 * 4 + 255) // 256 * 256 if expect > 1 else 0
        assert f(T, L, 64, 1) == uv + part, (L, T)
    # the same rule for dx's contraction over N (K = 64 is never split)
    T = 33
    uv = (2 * T * 4 + 255) // 256 * 256
    part = (expect * T * 64 * 4 + 255) // 256 * 256 if expect > 1 else 0
    assert f(T, 64, L, 1) == uv + part


def test_workspace_sizes(lib):
    f = lib.rlk_linear_logp_fwd_workspace_bytes
    assert f(0, 4096, 151936) == 0
    # one 16-byte record per (row, group of 256 columns), rounded to 256 B
    assert f(512, 4096, 151936) == 512 * (594 + 3) * 16  # virtual slices add <= 3 short groups
    # batches of at most 64 rows keep one record per 128-column half of a group
    assert f(3, 256, 1024) == 768  # 3 * (4 + 3) * 2 * 16 = 672, rounded up
    assert f(64, 4096, 151936) == 64 * 597 * 2 * 16
    assert f(65, 4096, 151936) == (65 * 597 * 16 + 255) // 256 * 256
    # the packed forward keeps two records per group for every T
    fp = lib.rlk_linear_logp_fwd_packed_workspace_bytes
    assert fp(512, 4096, 151936) == 512 * 597 * 2 * 16
    assert fp(3, 256, 1024) == f(3, 256, 1024)
    b = lib.rlk_linear_logp_bwd_workspace_bytes
    sizes = [b(T, 4096, 151936, 0, 1) for T in (1, 4, 64, 512, 5208)]
    assert all(x < y for x, y in zip(sizes, sizes[1:]))
    assert b(512, 4096, 151936, 0, 0) < b(512, 4096, 151936, 0, 1)
    assert b(0, 4096, 151936, 0, 1) == 0


# --------------------------------------------------------- host combine

def test_combine_host_matches_oracle():
    r = np.random.default_rng(5)
    T, H, V = 40, 16, 300
    h = r.standard_normal((T, H))
    W = r.standard_normal((V, H)) * 2.5   # peaky rows: small entropies
    y = r.integers(0, V, T)
    bounds = [0, 75, 150, 225, 300]
    parts = []
    for a, b in zip(bounds[:-1], bounds[1:]):
        m, R, B, zy = slice_partials_f64(h, W[a:b], y, a)
        parts.append(torch.tensor(np.stack([m, R, B, zy], axis=1), dtype=torch.float32))
    logp, ent, stats = rlk.combine_host(parts)
    full = forward_f64(h, W, y)
    assert np.abs(logp.numpy() - full["logp"]).max() <= 1e-5 * max(1, np.abs(full["logp"]).max())
    rel = np.abs(ent.numpy() - full["entropy"]) / np.maximum(np.abs(full["entropy"]), 1e-30)
    assert rel.max() <= 1e-4
    # the merged record finalises like the oracle's own merge
    acc = [p.double().numpy().T for p in parts]
    o = acc[0]
    for q in acc[1:]:
        o = merge_partials(o, q)
    fin = finalize_partials(o)
    np.testing.assert_allclose(stats.numpy()[:, 0], o[0], rtol=1e-6)
    np.testing.assert_allclose(logp.numpy(), fin["logp"], rtol=1e-5, atol=1e-5)


def test_combine_host_argument_errors(lib):
    assert lib.rlk_linear_logp_combine_host(P, 0, 4, NULL, NULL, NULL) == INVALID
    assert lib.rlk_linear_logp_combine_host(NULL, 2, 4, NULL, NULL, NULL) == INVALID
    assert lib.rlk_linear_logp_combine_host(NULL, 2, 0, NULL, NULL, NULL) == OK


def test_combine_host_empty_slice_and_missing_target():
    # slice 1 holds the target; a slice record with m = -inf (nothing) is neutral
    p0 = torch.tensor([[2.0, 0.5, -0.3, -math.inf]])
    p1 = torch.tensor([[3.0, 0.0, 0.0, 3.0]])
    logp, ent, st = rlk.combine_host([p0, p1])
    # by hand: base = p1 (larger max), d = -1, R = 0 + e^-1 (1.5), B = 0 + e^-1 (-0.3 + 1.5 * -1)
    e = math.exp(-1.0)
    R = e * 1.5
    B = e * (-0.3 - 1.5)
    assert math.isclose(st[0, 1].item(), R, rel_tol=1e-6)
    assert math.isclose(st[0, 2].item(), B, rel_tol=1e-6)
    assert math.isclose(logp[0].item(), -math.log1p(R), rel_tol=1e-6)
    assert math.isclose(ent[0].item(), math.log1p(R) - B / (1 + R), rel_tol=1e-6)


# ------------------------------------------------ allocation-free forward --

def fwd_na(lib, hidden=P, weight=P, targets=P, T=4, H=64, V=100, vs=0, vt=None, logp=P, ent=P,
           stats=P):
    vt = V if vt is None else vt
    return lib.rlk_linear_logp_fwd_noalloc(hidden, weight, targets, T, H, V, vs, vt, logp, ent,
                                           stats, NULL)


def scratch_bytes():
    txt = open(os.path.join(ROOT, "include", "rlk_linear.h")).read()
    m = re.search(r"#define RLK_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", txt)
    return int(m.group(1)) << int(m.group(2))


@pytest.mark.parametrize("kw,code", [
    (dict(T=-1), INVALID), (dict(H=96), SHAPE), (dict(vs=10, vt=105), INVALID),
    (dict(vs=5, vt=200, stats=P), INVALID), (dict(logp=NULL, ent=NULL, stats=NULL), INVALID),
    (dict(weight=NULL), INVALID), (dict(hidden=ctypes.c_void_p((1 << 20) + 2)), INVALID),
    # records of the tile path: T x (ceil(V/256) + 3) x 16 bytes > 8 MiB
    (dict(T=879, H=4096, V=151936), SCRATCH),
    # records of the streaming path: two per group
    (dict(T=64, H=64, V=1 << 20), SCRATCH),
])
def test_fwd_noalloc_argument_errors(lib, kw, code):
    assert fwd_na(lib, **kw) == code


def test_fwd_noalloc_limit_matches_the_workspace_query(lib):
    cap = scratch_bytes()
    assert cap == 8 << 20
    for T, V in [(878, 151936), (879, 151936), (64, 1000000), (1, (1 << 24) - 1)]:
        need = lib.rlk_linear_logp_fwd_workspace_bytes(T, 4096, V)
        st = fwd_na(lib, T=T, H=4096, V=V)
        assert (need <= cap) == (st != SCRATCH), (T, V, need, st)
    # within the limit, a valid call passes every check up to the device
    if not torch.cuda.is_available():
        assert fwd_na(lib, T=878, H=4096, V=151936) in (HIPERR, DEVICE)


def test_fwd_noalloc_T0_is_noop(lib):
    before = lib.rlk_call_count(6)
    assert fwd_na(lib, T=0, hidden=NULL, targets=NULL) == OK
    assert lib.rlk_call_count(6) == before + 1


# ------------------------------------------------------ dH slice merge --

def test_dh_merge_argument_errors(lib):
    raw = ctypes.CDLL(rlk.LIB_PATH)
    raw.rlk_linear_logp_dh_merge.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                             ctypes.c_int64, ctypes.c_void_p, ctypes.c_uint32,
                                             ctypes.c_void_p]
    m = raw.rlk_linear_logp_dh_merge
    assert m(P, 0, 4, 64, P, 0, NULL) == INVALID                   # no slices
    assert m(P, 1025, 4, 64, P, 0, NULL) == INVALID                # too many
    assert m(P, 2, -1, 64, P, 0, NULL) == INVALID
    assert m(P, 2, 4, 0, P, 0, NULL) == INVALID
    assert m(P, 2, 4, 64, P, 2, NULL) == INVALID                   # unknown flag
    assert m(P, 2, 4, 96, P, 0, NULL) == SHAPE                     # H not a multiple of 64
    assert m(NULL, 2, 4, 64, P, 0, NULL) == INVALID
    assert m(P, 2, 4, 64, ctypes.c_void_p((1 << 20) + 8), 0, NULL) == INVALID
    before = lib.rlk_call_count(7)
    assert m(NULL, 2, 0, 64, NULL, 0, NULL) == OK                  # T = 0: no-op
    assert lib.rlk_call_count(7) == before + 1
    if not torch.cuda.is_available():
        assert m(P, 2, 4, 64, P, 1, NULL) in (HIPERR, DEVICE)
