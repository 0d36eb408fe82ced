"""Seeded synthetic inputs for the linear log-prob — shared by tests, bench and smoke.

This module draws random numbers and rounds them to bf16; it holds none of the
operator's arithmetic, so both the CPU oracle and the HIP path may consume its
output. Everything is generated on the CPU with ``torch.Generator`` so the
bytes do not depend on the GPU. Draw order inside one case is fixed: hidden,
weight, targets, dlogp, dentropy.

Shapes follow the pages' workload: Qwen3-8B's LM head (H=4096, V=151936), the
actor run at TP=4 (a vocabulary slice of V/4 = 37984 rows), 5,208 packed
tokens per step and a 7,168-token response budget ("VIME Qwen3-8B TP4/CP2
200-round consistency experiment", section "Required gates"; "RL-Kernel
evidence h100-cp-gradient.json", ``runs[0].tokens``). The dataset and weights
behind those runs are not used; random inputs of the same shapes stand in.

Cases:
  tiny      T=64,  H=256,  V=1024; hidden N(0,1); W N(0,0.02^2); seed 0
  qwen512   T=512, H=4096, V=151936; hidden RMS-normalised N(0,1); W N(0,0.02^2); seed 1
  pool64    64 rows as qwen512 (seed 2) scored with qwen512's W; permutations
            from seeds 3/4/5; embedded in a T=512 batch drawn with seed 6
  step5208  T=5208 from 8 sequences of length U[256,1024] (seed 7)
  slice7168 T=7168, full W as qwen512 then x8 (exact: power of two), cut into
            4 slices of 37984 rows; targets over the full vocabulary; seed 8

LoRA linear (the page "RL-Kernel h3-runtime-integration-b200 report.json",
key ``lora_gate``: shapes N512 K384 T70, N2048 K1024 T257, N5120 K5120 T33;
rank 16 here, the page gives none): x N(0,1), W N(0,1/K), A N(0,1/K),
B N(0,1/r), dy N(0,1), all bf16; draw order x, W, A, B, dy; seeds 40, 41, 42.
"""

from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import torch

QWEN_H = 4096
QWEN_V = 151936
TP = 4
SLICE_V = QWEN_V // TP  # 37984
W_STD = 0.02
RMS_EPS = 1e-6


@dataclass
class Case:
    name: str
    hidden: torch.Tensor          # bf16 [T,H] (CPU)
    weight: torch.Tensor          # bf16 [V,H] (CPU)
    targets: torch.Tensor         # int32 [T] global vocabulary ids
    dlogp: torch.Tensor           # fp32 [T]
    dentropy: torch.Tensor | None  # fp32 [T] or None
    meta: dict = field(default_factory=dict)

    @property
    def T(self):
        return self.hidden.shape[0]

    @property
    def H(self):
        return self.hidden.shape[1]

    @property
    def V(self):
        return self.weight.shape[0]


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return g


def to_bf16(x: torch.Tensor) -> torch.Tensor:
    """Round-to-nearest-even fp32 -> bf16 (torch's conversion)."""
    return x.to(torch.bfloat16)


def rms_normalise(x: torch.Tensor) -> torch.Tensor:
    """x / sqrt(mean(x^2) + 1e-6) per row, fp32, no gain (input recipe only)."""
    x = x.float()
    return x * torch.rsqrt(x.pow(2).mean(dim=1, keepdim=True) + RMS_EPS)


def _hidden(g, T, H, rms):
    h = torch.randn(T, H, generator=g, dtype=torch.float32)
    return to_bf16(rms_normalise(h) if rms else h)


def _weight(g, V, H, std=W_STD, chunk_rows=8192):
    # drawn in row chunks of 8192 to bound the fp32 temporary
    out = torch.empty(V, H, dtype=torch.bfloat16)
    for r0 in range(0, V, chunk_rows):
        r1 = min(V, r0 + chunk_rows)
        out[r0:r1] = to_bf16(torch.randn(r1 - r0, H, generator=g, dtype=torch.float32) * std)
    return out


def make_case(name, T, H, V, seed, *, rms=True, w_scale=1, with_dentropy=True,
              target_range=None) -> Case:
    g = _gen(seed)
    hidden = _hidden(g, T, H, rms)
    weight = _weight(g, V, H)
    if w_scale != 1:
        # a power-of-two scale commutes with bf16 rounding, so this is exact
        assert w_scale in (2, 4, 8, 16)
        weight = weight * w_scale
    hi = V if target_range is None else target_range
    targets = torch.randint(0, hi, (T,), generator=g, dtype=torch.int64).to(torch.int32)
    dlogp = torch.randn(T, generator=g, dtype=torch.float32)
    dent = torch.randn(T, generator=g, dtype=torch.float32) if with_dentropy else None
    return Case(name, hidden, weight, targets, dlogp, dent, {"seed": seed, "rms": rms})


def tiny(seed=0) -> Case:
    return make_case("tiny", 64, 256, 1024, seed, rms=False)


_cache: dict = {}


def qwen512() -> Case:
    if "qwen512" not in _cache:
        _cache["qwen512"] = make_case("qwen512", 512, QWEN_H, QWEN_V, 1, with_dentropy=False)
    return _cache["qwen512"]


def qwen_rows(T: int, seed: int, V: int = QWEN_V):
    """hidden, targets, dlogp for T extra rows scored against an existing W."""
    g = _gen(seed)
    hidden = _hidden(g, T, QWEN_H, True)
    targets = torch.randint(0, V, (T,), generator=g, dtype=torch.int64).to(torch.int32)
    dlogp = torch.randn(T, generator=g, dtype=torch.float32)
    return hidden, targets, dlogp


def pool64():
    """The 64-row batch-invariance pool, its permutations and its embedding.

    Returns dict(hidden, targets, perms=[3 permutations], embed=dict(hidden,
    targets, positions)) where embed puts the pool rows at ``positions`` of a
    T=512 batch whose other rows are fresh draws.
    """
    if "pool64" not in _cache:
        hidden, targets, _ = qwen_rows(64, 2)
        perms = [torch.randperm(64, generator=_gen(s)) for s in (3, 4, 5)]
        g = _gen(6)
        pos = torch.randperm(512, generator=g)[:64]
        other = _hidden(g, 512, QWEN_H, True)
        other_t = torch.randint(0, QWEN_V, (512,), generator=g, dtype=torch.int64).to(torch.int32)
        other[pos] = hidden
        other_t[pos] = targets
        _cache["pool64"] = {"hidden": hidden, "targets": targets, "perms": perms,
                            "embed": {"hidden": other, "targets": other_t, "positions": pos}}
    return _cache["pool64"]


def step_lengths(total=5208, n=8, lo=256, hi=1024, seed=7):
    """8 sequence lengths in [lo, hi] summing to ``total`` (recorded only)."""
    g = _gen(seed)
    L = torch.randint(lo, hi + 1, (n,), generator=g).tolist()
    i = 0
    while sum(L) != total:
        step = 1 if sum(L) < total else -1
        if lo <= L[i % n] + step <= hi:
            L[i % n] += step
        i += 1
    return L


def step5208() -> Case:
    if "step5208" not in _cache:
        lengths = step_lengths()
        c = make_case("step5208", 5208, QWEN_H, QWEN_V, 7, with_dentropy=False)
        c.meta["seq_lengths"] = lengths
        _cache["step5208"] = c
    return _cache["step5208"]


def slice7168() -> Case:
    """Full-vocabulary case whose W is cut into TP=4 slices of 37984 rows."""
    if "slice7168" not in _cache:
        c = make_case("slice7168", 7168, QWEN_H, QWEN_V, 8, w_scale=8, with_dentropy=False)
        c.meta["slices"] = [(s * SLICE_V, (s + 1) * SLICE_V) for s in range(TP)]
        _cache["slice7168"] = c
    return _cache["slice7168"]


def digest(*tensors) -> str:
    """SHA-256 over the raw bytes of the given CPU tensors (input provenance)."""
    h = hashlib.sha256()
    for t in tensors:
        if t is None:
            continue
        t = t.contiguous()
        if t.dtype == torch.bfloat16:
            t = t.view(torch.int16)
        h.update(t.numpy().tobytes())
    return h.hexdigest()


def clear_cache():
    _cache.clear()


# ------------------------------------------------------------ LoRA linear ----

LORA_SHAPES = ((512, 384, 70), (2048, 1024, 257), (5120, 5120, 33))  # (N, K, T)
LORA_RANK = 16


@dataclass
class LoraCase:
    name: str
    x: torch.Tensor    # bf16 [T,K]
    W: torch.Tensor    # bf16 [N,K]
    A: torch.Tensor    # bf16 [r,K]
    B: torch.Tensor    # bf16 [N,r]
    dy: torch.Tensor   # bf16 [T,N]

    @property
    def T(self):
        return self.x.shape[0]

    @property
    def K(self):
        return self.x.shape[1]

    @property
    def N(self):
        return self.W.shape[0]

    @property
    def r(self):
        return self.A.shape[0]


def lora_case(N: int, K: int, T: int, seed: int, r: int = LORA_RANK) -> LoraCase:
    g = _gen(seed)
    x = to_bf16(torch.randn(T, K, generator=g))
    W = to_bf16(torch.randn(N, K, generator=g) / K ** 0.5)
    A = to_bf16(torch.randn(r, K, generator=g) / K ** 0.5)
    B = to_bf16(torch.randn(N, r, generator=g) / r ** 0.5)
    dy = to_bf16(torch.randn(T, N, generator=g))
    return LoraCase(f"lora_N{N}_K{K}_T{T}", x, W, A, B, dy)


def lora_page_cases():
    """The three shapes of the page's gate, seeds 40, 41, 42."""
    return [lora_case(N, K, T, 40 + i) for i, (N, K, T) in enumerate(LORA_SHAPES)]
