"""Builds librlk_linear.so in-tree with hipcc for gfx950.

    python -m rollout_rlk_linear_amd._build        (or: python rollout_rlk_linear_amd/_build.py)

Flags that matter for the bitwise contract:
  -ffp-contract=off   the arithmetic is exactly as written (no compiler-chosen
                      fused multiply-adds that could differ between kernels)
  -Xclang -target-feature -Xclang -packed-fp32-ops
                      no packed fp32 instructions
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "librlk_linear.so")
ARCH = "gfx950"

SOURCES = ["rlk_kernels.hip", "rlk_dh.hip", "rlk_microbench.hip", "rlk_lora.hip", "rlk_lora_fwd.hip",
           "rlk_abi.cpp"]
# Flags for one source only. The dH kernel's and the LoRA forward tile's
# translation units take the machine scheduler's iterative-ILP strategy: the
# same instructions, ordered so that dH runs 1-2% and the LoRA forward 3-7%
# faster; the logits' mainloop loses 3-6% and the small LoRA backwards up to
# 9% under it, so the rest keeps the default.
_ILP = ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"]
SOURCE_FLAGS = {"rlk_dh.hip": _ILP, "rlk_lora_fwd.hip": _ILP}
HEADERS = ["rlk_device.h", "rlk_internal.h", "rlk_lora_common.h"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def common_flags():
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function", "-Wno-inline-asm",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    cc = hipcc()
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src + ".o")
        cmd = [cc, *common_flags(), *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src),
               "-o", obj]
        if src.endswith(".cpp"):
            cmd[1:1] = ["-x", "hip"]
        _run(cmd, verbose)
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature: harmless notice
    err = "\n".join(line for line in r.stderr.splitlines()
                    if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


if __name__ == "__main__":
    print(build(verbose=True))
