"""Brute-force linear log-prob for tiny vocabularies — TEST INFRASTRUCTURE ONLY.

Pins the float64 oracle from outside float64. The logits of bf16 inputs are
dyadic rationals, so they are computed exactly with ``fractions.Fraction``;
exp and log are then evaluated with the ``decimal`` module at 50 significant
digits. Definitions are the plain softmax ones of the operator (page "VIME
Qwen3-8B TP4/CP2 200-round consistency experiment", section "User-facing
operator matrix": log-prob and entropy of the LM-head softmax):

    log p_v = z_v - log sum_u exp(z_u),  logp = log p_y,  entropy = -sum p log p.

Intended for V <= 64 and small H; cost is O(T V H) big-number operations.
"""

from __future__ import annotations

from decimal import Decimal, localcontext
from fractions import Fraction

import numpy as np

DIGITS = 50


def _frac_matrix(a64: np.ndarray):
    return [[Fraction(float(v)) for v in row] for row in np.asarray(a64, dtype=np.float64)]


def exact_logits(h64: np.ndarray, W64: np.ndarray):
    """z[t][v] = sum_k h[t,k] W[v,k] as exact Fractions (inputs exactly representable)."""
    hf = _frac_matrix(h64)
    Wf = _frac_matrix(W64)
    return [[sum((a * b for a, b in zip(hr, wr)), Fraction(0)) for wr in Wf] for hr in hf]


def _dec(fr: Fraction) -> Decimal:
    return Decimal(fr.numerator) / Decimal(fr.denominator)


def logp_entropy(h64: np.ndarray, W64: np.ndarray, y) -> tuple[list[Decimal], list[Decimal]]:
    """Per-row (logp, entropy) as 50-digit Decimals."""
    z = exact_logits(h64, W64)
    y = [int(v) for v in np.asarray(y)]
    logps, ents = [], []
    with localcontext() as ctx:
        ctx.prec = DIGITS + 10
        for zr, yt in zip(z, y):
            m = max(zr)
            d = [_dec(v - m) for v in zr]  # exact shift, then to Decimal
            e = [x.exp() for x in d]
            s = sum(e, Decimal(0))
            ls = s.ln()
            logp = [x - ls for x in d]
            ent = -sum((ei / s) * lp for ei, lp in zip(e, logp))
            logps.append(+logp[yt])
            ents.append(+ent)
    return logps, ents
