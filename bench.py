#!/usr/bin/env python3
"""Benchmark of the fused, batch-invariant linear log-prob on one MI355X.

One step = the whole hot path once: forward (logits tile + fixed-order
statistics + combine -> logp, entropy, stats) and backward (recompute, bf16
logit gradient, dW, split-K dH, ordered reduce -> dhidden bf16, dweight fp32)
over one batch of synthetic Qwen3-8B LM-head inputs (T = 512 tokens, H = 4096,
V = 151936; hidden RMS-normalised N(0,1), W N(0, 0.02^2), both bf16; uniform
targets; dlogp N(0,1)). Inputs are resident in HBM before the timed region.

Prints one JSON line: tokens/s over the timed steps, ms/step (also median with
a distribution-free 95% interval, and minimum, from per-step HIP events),
TFLOP/s (8 T H V flops per step) and the fraction of the bf16 dense MFMA
peak (published, and measured on the box by the library's microbenchmark);
the roofline of the dominant kernel (per-launch duration from HIP events the
library records on the launch stream); the other workloads (tiny, small-T
forward against the HBM roofline with a bitwise check, the 5208-token step,
one 37984-row vocabulary slice); the same GEMM shapes through torch.matmul
(hipBLASLt) as a yardstick; and the float64 CPU oracle timed on the same
batch.

    python bench.py [--steps 20] [--warmup 10] [--gpus 1] [--no-cpu-baseline] [--quick]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E, published
PUBLISHED_SCLK_GHZ = 2.4   # the clock the published peak assumes (256 CUs x 2.4 GHz x 4096 flop)
METRIC = "linear-logp fwd+bwd tokens/s and % bf16 MFMA peak at H4096 V151936 T512"
CSRC = os.path.join(ROOT, "rollout_rlk_linear_amd", "csrc")
from rollout_rlk_linear_amd._build import SOURCE_FLAGS  # noqa: E402  (per-source build flags)


# the sources that decide the linear-logp kernels' code and launches
HASHED_SOURCES = ("rlk_abi.cpp", "rlk_device.h", "rlk_internal.h", "rlk_kernels.hip", "rlk_dh.hip")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in HASHED_SOURCES:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
            h.update(repr(SOURCE_FLAGS.get(name, [])).encode())
    return h.hexdigest()[:16]


def load_traffic(kernel: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if current."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_hash") != kernel_source_hash():
        return None
    k = t.get("kernels", {}).get(kernel)
    return None if not k else k.get("hbm_bytes_per_launch")


def algorithmic_work(T, H, V, nsplits):
    """Per-step algorithmic flops and HBM bytes of each kernel: every operand
    read once and every output written once (G = the bf16 logit gradient
    [T][V], records 16 B per row and 256-column group, dH split partials fp32)."""
    G = -(-V // 256)
    f = 2.0 * T * H * V
    W, h, Gt = 2.0 * V * H, 2.0 * T * H, 2.0 * T * V
    return {
        "fwd_tile": (f, W + h + 16.0 * T * G),
        "bwd_recompute": (f, W + h + Gt),
        "bwd_dw": (f, Gt + h + 4.0 * V * H),
        "bwd_dh": (f, Gt + W + 4.0 * nsplits * T * H),
        "fwd_combine": (0.0, T * G * 16.0 + T * 4 * 6.0),
        "bwd_dh_reduce": (0.0, nsplits * T * H * 4.0 + T * H * 2.0),
    }


RIDGE = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)  # flop/B where the two roofs meet


def median_ci(xs):
    """Median, distribution-free ~95% interval of the median, minimum (ms)."""
    s = sorted(xs)
    n = len(s)
    med = s[n // 2] if n % 2 else 0.5 * (s[n // 2 - 1] + s[n // 2])
    half = 0.98 * math.sqrt(n)
    lo = max(0, int(math.floor(n / 2 - half)) - 1)
    hi = min(n - 1, int(math.ceil(n / 2 + half)))
    return {"median": round(med, 4), "ci95": [round(s[lo], 4), round(s[hi], 4)],
            "min": round(s[0], 4), "n": n}


def timed(torch, fn, warmup, steps):
    """Per-call HIP-event times (ms) on the current stream, and their total."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record()
    for i in range(steps):
        fn()
        ev[i + 1].record()
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    return per, ev[0].elapsed_time(ev[steps])


def graph_timed(torch, fn, outs, inner, reps):
    """GPU-side time per call (ms) of a short call: `inner` calls captured in
    one graph and replayed `reps` times, each replay timed by HIP events. Calls
    this short are issued faster by the GPU than by the Python loop that
    launches them, so per-call events from an eager loop would time the host.
    Every replay's outputs (the tensors in `outs`, written in place) must equal
    the eager call's bits. Returns (per-call times, bits equal on every replay)."""
    fn()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for _ in range(inner):
                fn()
    torch.cuda.synchronize()
    per, same = [], True
    for _ in range(reps):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1) / inner)
        same = same and all(torch.equal(o.view(torch.int16) if o.dtype == torch.bfloat16 else
                                        o.view(torch.int32), r.view(torch.int16)
                                        if r.dtype == torch.bfloat16 else r.view(torch.int32))
                            for o, r in zip(outs, ref))
    del g
    return per, same


def device_info(torch):
    p = torch.cuda.get_device_properties(0)
    info = {"name": p.name, "cu_count": p.multi_processor_count,
            "gcn_arch": getattr(p, "gcnArchName", None)}
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True,
                           timeout=20)
        if r.returncode == 0:
            d = json.loads(r.stdout)
            card = d[sorted(d)[0]]
            info["clocks"] = {k: v for k, v in card.items() if "clock" in k.lower()}
    except Exception as e:  # the clock readout is informative only
        info["clocks_error"] = type(e).__name__
    return info


def microbench(torch, rlk):
    """Measured denominators: HBM copy bandwidth and bf16 MFMA rate."""
    dev = torch.device("cuda:0")
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    per, _ = timed(torch, lambda: rlk.microbench_copy(dst, src), 2, 5)
    copy_gbs = 2 * n / (min(per) * 1e-3) / 1e9
    del src, dst
    sink = torch.zeros(4, dtype=torch.float32, device=dev)
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    wg, iters = 8 * ncu, 4096
    flops = [0.0]

    def mfma():
        flops[0] = rlk.microbench_mfma(sink, wg, iters)

    per, _ = timed(torch, mfma, 2, 5)
    mf = flops[0] / (min(per) * 1e-3) / 1e12
    # both MFMA shapes with the shader clock they ran at (in-kernel s_memtime
    # against the constant-rate wall clock)
    clocks = torch.zeros(2 * wg, dtype=torch.int64, device=dev)
    shapes = {}
    for shape, name in ((0, "16x16x32"), (1, "32x32x16")):
        info = {}

        def run():
            info["flops"], info["khz"] = rlk.microbench_mfma_clock(sink, clocks, wg, iters, shape)

        per_s, _ = timed(torch, run, 2, 5)
        c = clocks.view(wg, 2).double().sum(dim=0).cpu()
        sclk_ghz = float(c[0] / c[1]) * info["khz"] * 1e3 / 1e9
        tf = info["flops"] / (min(per_s) * 1e-3) / 1e12
        shapes[name] = {"TFLOPs": round(tf, 1), "sclk_GHz": round(sclk_ghz, 3),
                        "frac_published": round(tf / PEAK_BF16_TFLOPS, 4),
                        # the published peak scaled to the clock the run held
                        "frac_of_peak_at_that_clock": round(
                            tf / (PEAK_BF16_TFLOPS * sclk_ghz / PUBLISHED_SCLK_GHZ), 4)}
    del clocks
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    per_r, _ = timed(torch, lambda: rlk.microbench_read(src, sink, ncu), 2, 5)
    read_gbs = n / (min(per_r) * 1e-3) / 1e9
    del src
    # the vendor library's dense square GEMM as a second ceiling
    g = torch.Generator(device="cpu").manual_seed(12)
    a = torch.randn(8192, 8192, generator=g).to(torch.bfloat16).to(dev)
    b = torch.randn(8192, 8192, generator=g).to(torch.bfloat16).to(dev)
    per_g, _ = timed(torch, lambda: torch.matmul(a, b), 2, 5)
    gemm_tf = 2.0 * 8192 ** 3 / (min(per_g) * 1e-3) / 1e12
    del a, b
    torch.cuda.empty_cache()
    best = max(mf, gemm_tf, *(v["TFLOPs"] for v in shapes.values()))
    return {"copy_GBps": round(copy_gbs, 1), "copy_bytes": n, "read_GBps": round(read_gbs, 1),
            "read_bytes": n,
            "mfma_bf16_TFLOPs": round(mf, 1),
            "mfma_workgroups": wg, "mfma_iters": iters,
            "mfma_shapes": shapes,
            "hipblaslt_square_8192_bf16_TFLOPs": round(gemm_tf, 1),
            "measured_bf16_ceiling_TFLOPs": round(best, 1)}


def library_yardstick(torch, hidden, weight, kernels):
    """The same three GEMM shapes through torch.matmul (hipBLASLt on ROCm), as
    context for the per-kernel rates: the logits GEMM h W^T (bf16 logits
    written out, no softmax), dH = G W and dW = G^T h (bf16 out, and fp32 out
    where torch offers it), with G a random bf16 [T, V]. Only a yardstick:
    the library never calls it."""
    dev = hidden.device
    T, H = hidden.shape
    V = weight.shape[0]
    g = torch.Generator(device="cpu").manual_seed(11)
    G = torch.randn(T, V, generator=g).to(torch.bfloat16).to(dev)
    GT = G.t().contiguous()
    fl = 2.0 * T * H * V
    out = {"flops_per_gemm": fl, "T": T, "H": H, "V": V}
    cases = [("logits_hWt_bf16", lambda: torch.matmul(hidden, weight.t()), "fwd_tile"),
             ("dH_GW_bf16", lambda: torch.matmul(G, weight), "bwd_dh"),
             ("dW_GtH_bf16", lambda: torch.matmul(GT, hidden), "bwd_dw"),
             ("dW_GtH_fp32", lambda: torch.mm(GT, hidden, out_dtype=torch.float32), "bwd_dw")]
    for name, fn, ours in cases:
        try:
            per, _ = timed(torch, fn, 2, 5)
        except Exception as e:  # an op this torch build lacks is reported, not fatal
            out[name] = {"error": f"{type(e).__name__}: {str(e)[:120]}"}
            continue
        ms = sorted(per)[len(per) // 2]
        ent = {"ms": round(ms, 4), "tflops": round(fl / (ms * 1e-3) / 1e12, 1)}
        if ours in kernels:
            ent["library_kernel"] = ours
            ent["library_kernel_ms"] = round(kernels[ours]["avg_launch_ms"], 4)
        out[name] = ent
    del G, GT
    torch.cuda.empty_cache()
    return out


def to_dev(torch, c):
    dev = torch.device("cuda:0")
    return [x.to(dev).contiguous() for x in (c.hidden, c.weight, c.targets, c.dlogp)]


def workload_runs(torch, rlk, wl, read_gbs, steps):
    """The tiny case, small-T forwards (+ bitwise check), the 5208-token step
    and one vocabulary slice, timed on the GPU."""
    res = {}
    # tiny: launch-bound, for completeness
    c = wl.tiny()
    h, w, y, dl = to_dev(torch, c)
    de = c.dentropy.to("cuda:0")
    fo, bo = {}, {}

    def step1():
        o = rlk.fwd(h, w, y, out=fo)
        rlk.bwd(h, w, y, o["stats"], dl, de, out=bo)

    per, _ = timed(torch, step1, 3, steps)
    res["tiny_T64_H256_V1024"] = {"fwd_bwd_ms": median_ci(per), "dentropy": "N(0,1)"}

    # small T (rollout decode batches): the forward is a stream over W; bytes
    # 2HV + 2TH + 4T + 16T per call (W, hidden, targets, logp+entropy+stats).
    # Timed over W in its natural layout and over the packed copy (packed
    # once, its time reported apart). Bitwise check: every batch of T
    # consecutive rows of the 64-row pool, both layouts, against the same rows
    # inside the 512-row training batch (the tile path).
    c2w = wl.qwen512().weight.to("cuda:0")
    pool = wl.pool64()
    ph = pool["hidden"].to("cuda:0")
    pt = pool["targets"].to("cuda:0")
    emb = pool["embed"]
    pos = emb["positions"].to("cuda:0")
    H, V = c2w.shape[1], c2w.shape[0]
    train = rlk.fwd(emb["hidden"].to("cuda:0"), c2w, emb["targets"].to("cuda:0"))
    ref_bits = {k: train[k][pos].contiguous().view(torch.int32).clone()
                for k in ("logp", "entropy", "stats")}
    pw = rlk.pack_weight(c2w)
    per, _ = timed(torch, lambda: rlk.pack_weight(c2w, out=pw), 1, 5)
    small = {"pack_weight_ms": median_ci(per), "packed_bytes": int(pw.data.numel())}
    mismatches, compared = 0, 0
    for T in (1, 2, 3, 4, 16, 64):
        hh, tt = ph[:T].contiguous(), pt[:T].contiguous()
        byts = 2 * H * V + 2 * T * H + 20 * T + 8 * T
        row = {"bytes": byts}
        for name, fn in (("natural", lambda o: rlk.fwd(hh, c2w, tt, out=o)),
                         ("packed", lambda o: rlk.fwd_packed(hh, pw, tt, out=o))):
            fo = {}
            per, _ = timed(torch, lambda: fn(fo), 3, steps)
            ms = median_ci(per)
            gbs = byts / (ms["median"] * 1e-3) / 1e9
            row[name] = {"fwd_ms": ms, "GBps": round(gbs, 1),
                         "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
                         "frac_measured_read": round(gbs / read_gbs, 4) if read_gbs else None}
        small[f"T{T}"] = row
        for s0 in range(0, 64 - T + 1, T):
            hs, ts = ph[s0:s0 + T].contiguous(), pt[s0:s0 + T].contiguous()
            for o in (rlk.fwd(hs, c2w, ts), rlk.fwd_packed(hs, pw, ts)):
                for k in ("logp", "entropy", "stats"):
                    d = o[k].view(torch.int32) != ref_bits[k][s0:s0 + T]
                    mismatches += int(d.sum())
                    compared += d.numel()
    small["bitwise_vs_training_batch"] = {"mismatched_words": mismatches,
                                          "compared_words": compared}
    res["small_T_forward_H4096_V151936"] = small
    del c2w, pw, train

    # the entropy-regularised objective at T = 512: dlogp and dentropy both N(0,1)
    c = wl.qwen512()
    h, w, y, dl = to_dev(torch, c)
    de = torch.randn(c.T, generator=torch.Generator().manual_seed(14)).to("cuda:0")
    fo, bo = {}, {}

    def step_ent():
        o = rlk.fwd(h, w, y, out=fo)
        rlk.bwd(h, w, y, o["stats"], dl, de, out=bo)

    per, _ = timed(torch, step_ent, 3, steps)
    ms = median_ci(per)
    fl = 8.0 * c.T * c.H * c.V
    res["entropy_regularised_T512_H4096_V151936"] = {
        "fwd_bwd_ms": ms, "tokens_per_s": round(c.T / (ms["median"] * 1e-3), 1),
        "TFLOPs": round(fl / (ms["median"] * 1e-3) / 1e12, 1), "dentropy": "N(0,1), seed 14"}
    del h, w, y, dl, de, fo, bo

    # the 5208-token step (8 sequences), fwd+bwd
    c = wl.step5208()
    h, w, y, dl = to_dev(torch, c)
    fo, bo = {}, {}

    def step4():
        o = rlk.fwd(h, w, y, out=fo)
        rlk.bwd(h, w, y, o["stats"], dl, None, out=bo)

    per, _ = timed(torch, step4, 2, max(3, steps // 4))
    ms = median_ci(per)
    fl = 8.0 * c.T * c.H * c.V
    res["step_T5208_H4096_V151936"] = {
        "seq_lengths": c.meta.get("seq_lengths"), "fwd_bwd_ms": ms,
        "tokens_per_s": round(c.T / (ms["median"] * 1e-3), 1),
        "TFLOPs": round(fl / (ms["median"] * 1e-3) / 1e12, 1),
        "frac_bf16_peak": round(fl / (ms["median"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    del h, w, y, dl, fo, bo
    wl.clear_cache()

    # one TP=4 rank's vocabulary slice (rows 0..37983 of a W scaled by 8):
    # fwd (stats partials) + bwd with the global statistics, dH as fp32
    c = wl.slice7168()
    h, w, y, dl = to_dev(torch, c)
    a, b = c.meta["slices"][0]
    parts = [rlk.fwd(h, w[s0:s1].contiguous(), y, vocab_start=s0, vocab_total=c.V)["stats"]
             for s0, s1 in c.meta["slices"]]
    _, _, gstats = rlk.combine_host(parts)
    gstats = gstats.to("cuda:0")
    ws = w[a:b].contiguous()
    del w, parts
    fo, bo = {}, {}

    def step5():
        rlk.fwd(h, ws, y, vocab_start=a, vocab_total=c.V, out=fo)
        rlk.bwd(h, ws, y, gstats, dl, None, vocab_start=a, vocab_total=c.V, dhidden_f32=True,
                out=bo)

    per, _ = timed(torch, step5, 2, max(3, steps // 4))
    ms = median_ci(per)
    Vs = b - a
    fl = 8.0 * c.T * c.H * Vs
    res["slice_T7168_H4096_V37984"] = {
        "fwd_bwd_ms": ms, "tokens_per_s": round(c.T / (ms["median"] * 1e-3), 1),
        "TFLOPs": round(fl / (ms["median"] * 1e-3) / 1e12, 1),
        "frac_bf16_peak": round(fl / (ms["median"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    wl.clear_cache()

    # LoRA linear on the three shapes of the runtime report's gate (rank 16,
    # scale 2): forward, and forward + full backward (dx, dA, dB). Base-product
    # flops 2TKN per product (fwd 1, fwd+bwd 2); bytes of W per product.
    lora = {}
    for c in wl.lora_page_cases():
        x, W, A, B, dy = (t.to("cuda:0").contiguous() for t in (c.x, c.W, c.A, c.B, c.dy))
        yb = torch.empty(c.T, c.N, dtype=torch.bfloat16, device="cuda:0")
        ws = torch.empty(max(256, rlk.load_library().rlk_lora_linear_workspace_bytes(
            c.T, c.K, c.N, c.r)), dtype=torch.uint8, device="cuda:0")
        dxb = torch.empty(c.T, c.K, dtype=torch.bfloat16, device="cuda:0")
        dab = torch.empty(c.r, c.K, dtype=torch.float32, device="cuda:0")
        dbb = torch.empty(c.N, c.r, dtype=torch.float32, device="cuda:0")

        def fwd_bwd():
            rlk.lora_fwd(x, W, A, B, 2.0, out=yb, ws=ws)
            rlk.lora_bwd(x, W, A, B, dy, 2.0, ws=ws, out=(dxb, dab, dbb))

        # eager per-call events (host-paced for calls this short), then the
        # GPU-side time from replayed graphs, which the roofline uses
        per_fe, _ = timed(torch, lambda: rlk.lora_fwd(x, W, A, B, 2.0, out=yb, ws=ws), 3, steps)
        per_f, same_f = graph_timed(torch, lambda: rlk.lora_fwd(x, W, A, B, 2.0, out=yb, ws=ws),
                                    [yb], 20, steps)
        per_b, same_b = graph_timed(torch, fwd_bwd, [yb, dxb, dab, dbb], 20, steps)
        mf, mb = median_ci(per_f), median_ci(per_b)
        wbytes = 2 * c.N * c.K
        # algorithmic work of the forward: every operand read once, y written once
        fbytes = wbytes + 2 * c.r * (c.K + c.N) + 2 * c.T * c.K + 2 * c.T * c.N
        fflops = 2 * c.T * c.K * c.N + 2 * c.T * c.r * (c.K + c.N)
        secs = mf["median"] * 1e-3
        ai = fflops / fbytes
        bound = "mfma" if ai >= RIDGE else "hbm"
        achieved = (fflops / secs / 1e12) if bound == "mfma" else (fbytes / secs / 1e9)
        peak = PEAK_BF16_TFLOPS if bound == "mfma" else PEAK_HBM_GBS
        lora[c.name] = {"rank": c.r, "fwd_ms": mf, "fwd_bwd_ms": mb,
                        "timing": "graph of 20 calls replayed (GPU-side time per call)",
                        "graph_replays_bit_equal": bool(same_f and same_b),
                        "fwd_ms_eager_per_call_events": median_ci(per_fe),
                        "fwd_W_GBps": round(wbytes / secs / 1e9, 1),
                        "fwd_TFLOPs": round(2 * c.T * c.K * c.N / secs / 1e12, 2),
                        "fwd_roofline": {"bound": bound, "bytes": fbytes, "flops": fflops,
                                         "flop_per_byte": round(ai, 1),
                                         "achieved": round(achieved, 1),
                                         "unit": "TFLOP/s" if bound == "mfma" else "GB/s",
                                         "peak": peak, "frac": round(achieved / peak, 4)}}
    res["lora_gate_shapes"] = lora
    return res


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(case, rows: int, tiny=None):
    """The float64 oracle (unchanged) on the first ``rows`` tokens of the batch,
    and on the whole tiny case (T=64, H=256, V=1024) when given."""
    from threadpoolctl import threadpool_info

    from oracle import backward, forward

    def run(c, n):
        h = c.hidden[:n].contiguous()
        y = c.targets[:n].contiguous()
        dl = c.dlogp[:n].contiguous()
        t0 = time.perf_counter()
        forward(h, c.weight, y)
        backward(h, c.weight, y, dl, None)
        return time.perf_counter() - t0

    # the oracle on the same sample until about 10 s of CPU work is timed
    dt, reps = 0.0, 0
    while reps < 6 and (reps == 0 or dt < 10.0):
        dt += run(case, rows)
        reps += 1
    pools = threadpool_info()
    threads = max([p.get("num_threads", 1) for p in pools] or [1])
    blas = [{k: p.get(k) for k in ("internal_api", "version", "num_threads", "threading_layer")}
            for p in pools if p.get("user_api") == "blas"]
    what = "the whole batch" if rows == case.T else f"the first {rows} of the {case.T} tokens"
    out = {"value": rows * reps / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": f"{what}, full vocabulary, float64 forward + backward (all of dH and dW), "
                     f"{reps} run{'s' if reps > 1 else ''}; {dt:.1f} s wall",
           "cpu_model": cpu_model(), "host_cpus": len(os.sched_getaffinity(0)), "blas": blas}
    if tiny is not None:
        run(tiny, tiny.T)  # warm-up: the first call pays the BLAS start-up
        dtt = run(tiny, tiny.T)
        out["tiny_T64_H256_V1024"] = {"value": tiny.T / dtt, "unit": "tokens/s",
                                      "wall_s": round(dtt, 5)}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=512)
    ap.add_argument("--quick", action="store_true",
                    help="only the T=512 step (no microbenchmarks, other workloads or clocks)")
    ap.add_argument("--out", default=None, help="also append the JSON line to this file")
    ap.add_argument("--profile-case", choices=["fwd_t1", "fwd_t64", "fwd_packed_t1", "fwd_packed_t64", "read",
                                               "mfma16", "mfma32", "lora"],
                    default=None,
                    help="run only this case's calls (warmup + steps), for profilers: fwd_t1 / _t64 = "
                         "the forward of 1 / 64 rows over the full vocabulary (natural layout), "
                         "fwd_packed_t1 / _t64 = the same over the packed weight with 1 / 64 rows, "
                         "read = the 1 GiB streaming-read microbenchmark, mfma16 / mfma32 = the "
                         "clocked MFMA-rate kernel in the 16x16x32 / 32x32x16 shape, lora = the "
                         "LoRA-linear forward and backward on the runtime report's three shapes")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain 1 GiB device-to-device copy (3 times), the reference "
                         "for scaling the FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU (asked for --gpus {args.gpus}, WORLD_SIZE "
              f"{world}); the library has no multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import torch

    import rollout_rlk_linear_amd as rlk
    import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "copies": 3}), flush=True)
        return
    rlk.load_library()
    c = wl.qwen512()
    if args.profile_case == "read":
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0").fill_(1)
        sink = torch.zeros(4, dtype=torch.float32, device="cuda:0")
        ncu = torch.cuda.get_device_properties(0).multi_processor_count
        per, _ = timed(torch, lambda: rlk.microbench_read(src, sink, ncu), args.warmup, args.steps)
        print(json.dumps({"profile_case": "read", "ms": median_ci(per)}), flush=True)
        return
    if args.profile_case == "lora":
        for lc in wl.lora_page_cases():
            x, W, A, B, dy = (t.to("cuda:0").contiguous() for t in (lc.x, lc.W, lc.A, lc.B, lc.dy))
            per, _ = timed(torch, lambda: (rlk.lora_fwd(x, W, A, B, 2.0),
                                           rlk.lora_bwd(x, W, A, B, dy, 2.0)), args.warmup, args.steps)
            print(json.dumps({"profile_case": "lora", "shape": lc.name, "fwd_bwd_ms": median_ci(per)}),
                  flush=True)
        return
    if args.profile_case in ("mfma16", "mfma32"):
        ncu = torch.cuda.get_device_properties(0).multi_processor_count
        wg, iters = 8 * ncu, 4096
        sink = torch.zeros(4, dtype=torch.float32, device="cuda:0")
        clocks = torch.zeros(2 * wg, dtype=torch.int64, device="cuda:0")
        shape = 0 if args.profile_case == "mfma16" else 1
        info = {}

        def run():
            info["flops"], info["khz"] = rlk.microbench_mfma_clock(sink, clocks, wg, iters, shape)

        per, _ = timed(torch, run, args.warmup, args.steps)
        cs = clocks.view(wg, 2).double().sum(dim=0).cpu()
        print(json.dumps({"profile_case": args.profile_case, "ms": median_ci(per),
                          "TFLOPs": info["flops"] / (min(per) * 1e-3) / 1e12,
                          "sclk_GHz": float(cs[0] / cs[1]) * info["khz"] * 1e-6}), flush=True)
        return
    if args.profile_case is not None:
        w = c.weight.to("cuda:0")
        pool = wl.pool64()
        nrow = 64 if args.profile_case.endswith("t64") else 1
        h1, y1 = pool["hidden"][:nrow].to("cuda:0"), pool["targets"][:nrow].to("cuda:0")
        fo1 = {}
        if args.profile_case in ("fwd_t1", "fwd_t64"):
            fn = lambda: rlk.fwd(h1, w, y1, out=fo1)  # noqa: E731
        else:
            pw = rlk.pack_weight(w)
            fn = lambda: rlk.fwd_packed(h1, pw, y1, out=fo1)  # noqa: E731
        per, _ = timed(torch, fn, args.warmup, args.steps)
        print(json.dumps({"profile_case": args.profile_case, "fwd_ms": median_ci(per)}), flush=True)
        return
    T, H, V = c.T, c.H, c.V
    hidden, weight, targets, dlogp = to_dev(torch, c)
    fo, bo = {}, {}

    def step():
        o = rlk.fwd(hidden, weight, targets, out=fo)
        rlk.bwd(hidden, weight, targets, o["stats"], dlogp, None, out=bo)

    # warm-up: the clock takes about ten steps to settle after the idle set-up
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # headline pass: the K steps between two events, nothing recorded between
    # them (an event between steps adds a few microseconds to each boundary)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    e0.record()
    for i in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_total = e0.elapsed_time(e1)
    ms_step = ms_total / args.steps
    # second pass: an event after every step, for the distribution of step times
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    ev[0].record()
    for i in range(args.steps):
        step()
        ev[i + 1].record()
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]
    # third pass, for the per-kernel table: the library's per-launch events
    rlk.profile_begin()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    prof = rlk.profile_end()
    prof_per_step = sum(ms for ms, _ in prof.values()) / args.steps
    tokens_s = T * args.steps / (ms_total / 1e3)
    flops_step = 8.0 * T * H * V
    tflops = flops_step / (ms_step / 1e3) / 1e12

    nsplits = max(1, min(8, V // 16384))
    launches = {k: n // args.steps for k, (_, n) in prof.items() if n}
    work = algorithmic_work(T, H, V, nsplits)
    kernels = {}
    for k, (ms, n) in prof.items():
        if n == 0:
            continue
        fl, by = work.get(k, (0.0, 0.0))
        nl = max(1, launches[k])
        fl_l, by_l = fl / nl, by / nl
        avg_s = ms / n / 1e3
        ai = fl_l / by_l if by_l else None
        kernels[k] = {"ms_per_step": ms / args.steps, "launches_per_step": launches[k],
                      "avg_launch_ms": ms / n, "flops_per_launch": fl_l, "bytes_per_launch": by_l,
                      "flop_per_byte": round(ai, 1) if ai else None,
                      "bound": "mfma" if fl_l and ai >= RIDGE else "hbm",
                      "tflops": fl_l / avg_s / 1e12, "gbs": by_l / avg_s / 1e9}
    dom = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
    dk = kernels[dom]
    if dk["bound"] == "mfma":
        roof = {"bound": "mfma", "achieved": round(dk["tflops"], 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(dk["tflops"] / PEAK_BF16_TFLOPS, 4)}
    else:
        roof = {"bound": "hbm", "achieved": round(dk["gbs"], 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(dk["gbs"] / PEAK_HBM_GBS, 4)}
    roof["kernel"] = dom
    roof["avg_launch_ms"] = round(dk["avg_launch_ms"], 4)
    roof["flop_per_byte"] = dk["flop_per_byte"]
    roof["ridge_flop_per_byte"] = round(RIDGE, 1)
    roof["tflops"] = round(dk["tflops"], 2)
    roof["traffic"] = load_traffic(dom)

    result = {
        "metric": METRIC, "value": round(tokens_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "Qwen3-8B LM head linear-logp fwd+bwd, T=512 H=4096 V=151936",
                   "T": T, "H": H, "V": V, "seed": 1, "dlogp": "N(0,1)", "dentropy": None,
                   "parallelism": "none (1 GPU)",
                   "inputs_sha256": wl.digest(c.hidden, c.weight, c.targets)[:16]},
        "step_ms": median_ci(per),
        "tflops": round(tflops, 2), "frac_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "model_tflops_6thv": round(0.75 * tflops, 2),
        "wall_s_timed": round(wall, 4),
        "kernel_pass_ms_per_step": round(prof_per_step, 4),
        "kernels": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                    for k, v in kernels.items()},
        "roofline": roof,
        "backend": rlk.backend_id(),
        "kernel_source": kernel_source_hash(),
    }
    del fo, bo
    if not args.quick:
        result["device"] = device_info(torch)
        result["hipblaslt_yardstick"] = library_yardstick(torch, hidden, weight, kernels)
        mb = microbench(torch, rlk)
        result["microbench"] = mb
        result["frac_measured_mfma"] = round(tflops / mb["mfma_bf16_TFLOPs"], 4)
        result["frac_measured_ceiling"] = round(tflops / mb["measured_bf16_ceiling_TFLOPs"], 4)
        result["workloads"] = workload_runs(torch, rlk, wl, mb["read_GBps"], args.steps)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl.qwen512(), min(args.cpu_rows, T), wl.tiny())
    else:
        result["cpu_baseline"] = None
    line = json.dumps(result)
    print(line, flush=True)
    if args.out:
        with open(args.out, "a") as f:
            f.write(line + "\n")


if __name__ == "__main__":
    main()
