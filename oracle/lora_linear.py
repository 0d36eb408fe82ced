"""float64 CPU oracle of the LoRA linear — TEST INFRASTRUCTURE ONLY.

Imported only by tests, ``__graft_entry__.smoke()`` and bench.py's CPU
baseline; never by the product path, and it imports nothing from it.

Source: the page "RL-Kernel h3-runtime-integration-b200 report.json", key
``lora_gate``. Its three entries check a linear layer whose base weight is
frozen (``base_frozen``) and that carries a trainable low-rank adapter, on
shapes "N512 K384 T70", "N2048 K1024 T257" and "N5120 K5120 T33" (N output
features, K input features, T tokens). Each entry reports that the layer is
``repeatable`` and ``forward_rows_independent``, and the norm-wise relative
error against float64 of the forward output and of the gradients of the
input x and of the two adapter factors A and B (``forward_rel_err_vs_fp64``,
``grad_x_rel_err_vs_fp64``, ``grad_a_rel_err_vs_fp64``,
``grad_b_rel_err_vs_fp64``).

The page gives no formula. The plainest reading of a low-rank adapter on a
frozen linear (the merged weight W + s B A) is, per token row x_t in R^K,

    y_t = W x_t + s B (A x_t)       W in R^{N x K}, A in R^{r x K}, B in R^{N x r}

with a scalar scale s (the adapter's alpha / r; 1 when absent). With
u = x A^T (the adapter's rank-r code of each row) and an output gradient dy,
calculus gives

    dx = dy W + s (dy B) A       dA = s (dy B)^T x       dB = s dy^T u

and no gradient for the frozen W. ``rel_err`` is the page's norm-wise error:
||a - ref||_F / ||ref||_F.

Inputs arrive as bf16 (x, W, A, B, dy) and are decoded exactly to float64;
everything after that is float64.
"""

from __future__ import annotations

import numpy as np

from .linear_logp import _as_f64


def lora_forward(x, W, A, B, scale: float = 1.0) -> dict:
    """y = x W^T + s (x A^T) B^T, and u = x A^T (float64)."""
    x64, W64, A64, B64 = (_as_f64(t) for t in (x, W, A, B))
    u = x64 @ A64.T
    y = x64 @ W64.T + float(scale) * (u @ B64.T)
    return {"y": y, "u": u}


def lora_backward(x, W, A, B, dy, scale: float = 1.0) -> dict:
    """dx = dy W + s (dy B) A, dA = s (dy B)^T x, dB = s dy^T (x A^T) (float64)."""
    x64, W64, A64, B64, dy64 = (_as_f64(t) for t in (x, W, A, B, dy))
    s = float(scale)
    v = dy64 @ B64          # [T, r]: the output gradient seen through B
    u = x64 @ A64.T         # [T, r]
    return {"dx": dy64 @ W64 + s * (v @ A64), "dA": s * (v.T @ x64), "dB": s * (dy64.T @ u)}


def rel_err(a, ref) -> float:
    """Norm-wise relative error ||a - ref||_F / ||ref||_F (float64)."""
    a64 = np.asarray(_as_f64(a), dtype=np.float64)
    r64 = np.asarray(_as_f64(ref), dtype=np.float64)
    return float(np.linalg.norm(a64 - r64) / np.linalg.norm(r64))
