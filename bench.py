#!/usr/bin/env python3
"""Benchmark of the fused, batch-invariant linear log-prob on one MI355X.

One step = the whole hot path once: forward (logits tile + fixed-order
statistics + combine -> logp, entropy, stats) and backward (recompute, bf16
logit gradient, dW, split-K dH, ordered reduce -> dhidden bf16, dweight fp32)
over one batch of synthetic Qwen3-8B LM-head inputs (T = 512 tokens, H = 4096,
V = 151936; hidden RMS-normalised N(0,1), W N(0, 0.02^2), both bf16; uniform
targets; dlogp N(0,1)). Inputs are resident in HBM before the timed region.

Prints one JSON line: tokens/s, ms/step, TFLOP/s (8 T H V flops per step) and
fraction of the bf16 dense MFMA peak, the roofline of the dominant kernel
(per-launch duration measured with HIP events recorded by the library on the
launch stream), and the float64 CPU oracle timed on a bounded sample.

    python bench.py [--steps 20] [--warmup 3] [--gpus 1] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E, published
METRIC = "linear-logp fwd+bwd tokens/s and % bf16 MFMA peak at H4096 V151936 T512"
MFMA_KERNELS = ("fwd_tile", "bwd_recompute", "bwd_dw", "bwd_dh")
CSRC = os.path.join(ROOT, "rollout_rlk_linear_amd", "csrc")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, launch_bytes_alg: float):
    """HBM bytes per launch from committed rocprofv3 counter runs, if current."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_hash") != kernel_source_hash():
        return None
    k = t.get("kernels", {}).get(kernel)
    if not k:
        return None
    return k.get("hbm_bytes_per_launch")


def algorithmic_work(T, H, V, nchunks, nsplits):
    """Per-step algorithmic flops (MFMA kernels) and bytes (the others)."""
    G = -(-V // 256)
    f = 2.0 * T * H * V
    return {
        "fwd_tile": ("flops", f),
        "bwd_recompute": ("flops", f),
        "bwd_dw": ("flops", f),
        "bwd_dh": ("flops", f),
        "fwd_combine": ("bytes", T * G * 16 + T * 4 * 6),
        "bwd_rowprep": ("bytes", T * (16 + 12 + 32)),
        "bwd_dh_reduce": ("bytes", nsplits * T * H * 4 + T * H * 2),
    }


def cpu_baseline(case, rows: int):
    """The float64 oracle (unchanged) on the first ``rows`` tokens of the batch."""
    import numpy as np  # noqa: F401
    from threadpoolctl import threadpool_info

    from oracle import backward, forward

    h = case.hidden[:rows].contiguous()
    y = case.targets[:rows].contiguous()
    dl = case.dlogp[:rows].contiguous()
    t0 = time.perf_counter()
    forward(h, case.weight, y)
    backward(h, case.weight, y, dl, None)
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    return {"value": rows / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {rows} of the {case.T} tokens, full vocabulary, float64 forward + "
                      f"backward (all of dH and dW for the sample); {dt:.1f} s wall"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=512)
    ap.add_argument("--out", default=None, help="also append the JSON line to this file")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain 1 GiB device-to-device copy (3 times), the reference "
                         "for scaling the FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU (asked for --gpus {args.gpus}, WORLD_SIZE "
              f"{world}); the multi-GPU path is not part of this build", file=sys.stderr)
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
    T, H, V = c.T, c.H, c.V
    dev = torch.device("cuda:0")
    hidden, weight, targets = (x.to(dev).contiguous() for x in (c.hidden, c.weight, c.targets))
    dlogp = c.dlogp.to(dev).contiguous()
    fo, bo = {}, {}

    def step():
        o = rlk.fwd(hidden, weight, targets, out=fo)
        rlk.bwd(hidden, weight, targets, o["stats"], dlogp, None, out=bo)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    rlk.profile_begin()
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    prof = rlk.profile_end()
    ms_total = e0.elapsed_time(e1)
    ms_step = ms_total / args.steps
    tokens_s = T * args.steps / (ms_total / 1e3)
    flops_step = 8.0 * T * H * V
    tflops = flops_step / (ms_step / 1e3) / 1e12

    # plan figures for the per-launch work
    nsplits = max(1, min(8, V // 16384))
    launches = {k: n // args.steps for k, (_, n) in prof.items() if n}
    work = algorithmic_work(T, H, V, launches.get("bwd_recompute", 1), nsplits)
    kernels = {}
    for k, (ms, n) in prof.items():
        if n == 0:
            continue
        kind, per_step = work.get(k, ("bytes", 0.0))
        per_launch = per_step / max(1, launches[k])
        avg_s = ms / n / 1e3
        rate = per_launch / avg_s / (1e12 if kind == "flops" else 1e9)
        kernels[k] = {"ms_per_step": ms / args.steps, "launches_per_step": launches[k],
                      "avg_launch_ms": ms / n, "kind": kind, "work_per_launch": per_launch,
                      ("tflops" if kind == "flops" else "gbs"): rate}
    dom = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
    dk = kernels[dom]
    if dk["kind"] == "flops":
        roof = {"bound": "mfma", "achieved": round(dk["tflops"], 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(dk["tflops"] / PEAK_BF16_TFLOPS, 4)}
    else:
        roof = {"bound": "hbm", "achieved": round(dk["gbs"], 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(dk["gbs"] / PEAK_HBM_GBS, 4)}
    roof["kernel"] = dom
    roof["avg_launch_ms"] = round(dk["avg_launch_ms"], 4)
    roof["traffic"] = load_traffic(dom, dk["work_per_launch"])

    result = {
        "metric": METRIC, "value": round(tokens_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "Qwen3-8B LM head linear-logp fwd+bwd, T=512 H=4096 V=151936",
                   "T": T, "H": H, "V": V, "seed": 1, "dlogp": "N(0,1)", "dentropy": None,
                   "parallelism": "none (1 GPU)",
                   "inputs_sha256": wl.digest(c.hidden, c.weight, c.targets)[:16]},
        "tflops": round(tflops, 2), "frac_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "wall_s_timed": round(wall, 4),
        "kernels": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                    for k, v in kernels.items()},
        "roofline": roof,
        "backend": rlk.backend_id(),
        "kernel_source": kernel_source_hash(),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(c, min(args.cpu_rows, T))
    else:
        result["cpu_baseline"] = None
    line = json.dumps(result)
    print(line, flush=True)
    if args.out:
        with open(args.out, "a") as f:
            f.write(line + "\n")


if __name__ == "__main__":
    main()
