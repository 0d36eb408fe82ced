"""float64 CPU oracle of the fused linear log-prob — TEST INFRASTRUCTURE ONLY.

Imported only by tests, ``__graft_entry__.smoke()`` and bench.py's CPU
baseline; never by the product path, and it imports nothing from it.

The operator (page "VIME Qwen3-8B TP4/CP2 200-round consistency experiment",
section "User-facing operator matrix": the strict linear-logp provider replaces
VIME's ``calculate_log_probs_and_entropy``) maps, per token t,

    hidden h_t in R^H,  LM-head weight W in R^{V x H},  target id y_t

to the plain softmax quantities of the logits z_t = W h_t:

    log p_{t,v} = z_{t,v} - log sum_u exp(z_{t,u})
    logp_t      = log p_{t,y_t}
    entropy_t   = - sum_v p_{t,v} log p_{t,v}            (nats)

The page fixes no temperature other than 1 (section "Required gates"), no bias
and no scale, so none is applied. Inputs arrive as bf16 bit patterns and are
decoded exactly to float64; everything after that is float64.

Numerical form (no change of value, only of rounding): log-sum-exp is taken
relative to the row maximum m_t, with the lowest index v* attaining it held
out, R_t = sum_{v != v*} exp(z_{t,v} - m_t), so log sum exp(z - m) = log1p(R)
keeps full relative accuracy when the softmax is peaky (R << 1).

The backward pass is the derivative of the two outputs. The evidence page
"RL-Kernel evidence h100-cp-gradient.json" (``validation.runtime_readbacks``,
module ``logp`` under ``megatron/training``) shows the op inside the training
framework whose actor-train phase back-propagates through it; the gradient is
fixed by calculus:

    d logp_t / d z_{t,v}    = [v == y_t] - p_{t,v}
    d entropy_t / d z_{t,v} = -p_{t,v} (log p_{t,v} + entropy_t)

    G_{t,v} = dlogp_t ([v == y_t] - p_{t,v}) - dent_t p_{t,v} (log p_{t,v} + entropy_t)
    dH = G W,    dW = G^T h.

Vocabulary slices (one GPU's share of a tensor-parallel LM head; the page's
"Required gates" run the actor at TP=4): a slice [a, a+Vs) reports the
partial (m_s, R_s, B_s, zy_s) with B_s = sum_v exp(z_v - m_s)(z_v - m_s) and
zy_s = z_{y} if a <= y < a+Vs else -inf. ``merge_partials`` is the algebra
that combines two such partials; ``finalize_partials`` turns a whole-vocabulary
partial into logp and entropy. Combining over any partition of the vocabulary
reproduces ``forward_f64`` (pinned in the tests).

Rows are processed in blocks so that a [block, V] float64 logit tile is the
largest temporary.
"""

from __future__ import annotations

import numpy as np

ROW_BLOCK = 256


# --------------------------------------------------------------------------
# bf16 decoding (exact)
# --------------------------------------------------------------------------

def decode_bf16(x) -> np.ndarray:
    """bf16 values -> float64, exactly.

    ``x`` is either a torch ``bfloat16`` tensor (CPU) or a numpy ``uint16``
    array of raw bf16 bit patterns. A bf16 number is the top 16 bits of an
    IEEE binary32, so shifting the pattern left by 16 gives the float32 with
    the same value, and float32 -> float64 is exact.
    """
    if hasattr(x, "dtype") and str(getattr(x, "dtype", "")) == "torch.bfloat16":
        import torch

        bits = x.contiguous().view(torch.int16).numpy().view(np.uint16)
    else:
        bits = np.asarray(x)
        if bits.dtype != np.uint16:
            raise TypeError("decode_bf16 expects a torch.bfloat16 tensor or uint16 bits")
    f32 = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return f32.astype(np.float64)


def _as_f64(x) -> np.ndarray:
    if hasattr(x, "dtype") and str(getattr(x, "dtype", "")) == "torch.bfloat16":
        return decode_bf16(x)
    if hasattr(x, "numpy"):
        x = x.detach().cpu().numpy()
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return decode_bf16(x)
    return x.astype(np.float64)


def _as_index(y) -> np.ndarray:
    if hasattr(y, "numpy"):
        y = y.detach().cpu().numpy()
    return np.asarray(y).astype(np.int64)


# --------------------------------------------------------------------------
# per-block softmax statistics (plain definitions)
# --------------------------------------------------------------------------

def _row_stats(z: np.ndarray):
    """Max, held-out argmax and R for each row of a float64 logit block.

    m = max_v z; v* = lowest index attaining m; R = sum_{v != v*} exp(z - m).
    Returns (m, vstar, R, d) with d = z - m.
    """
    m = z.max(axis=1)
    vstar = z.argmax(axis=1)  # numpy returns the first (lowest) index of the max
    d = z - m[:, None]
    e = np.exp(d)
    e[np.arange(z.shape[0]), vstar] = 0.0
    R = e.sum(axis=1)
    return m, vstar, R, d


def _log_softmax_block(z: np.ndarray):
    """log p for a block of logits, plus m, R, log-normaliser relative to m."""
    m, vstar, R, d = _row_stats(z)
    lz = np.log1p(R)  # log sum_v exp(z_v - m)
    logp_all = d - lz[:, None]
    return logp_all, m, R, lz


# --------------------------------------------------------------------------
# forward
# --------------------------------------------------------------------------

def forward_f64(h: np.ndarray, W: np.ndarray, y: np.ndarray, row_block: int = ROW_BLOCK):
    """Full-vocabulary forward in float64.

    h [T,H], W [V,H] (float64), y [T] ints in [0, V).
    Returns dict with logp[T], entropy[T], lse[T], m[T], R[T].
    """
    h = np.asarray(h, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    y = _as_index(y)
    T = h.shape[0]
    V = W.shape[0]
    if T and (y.min() < 0 or y.max() >= V):
        raise ValueError("targets must lie in [0, V)")
    out = {k: np.empty(T) for k in ("logp", "entropy", "lse", "m", "R")}
    for r0 in range(0, T, row_block):
        r1 = min(T, r0 + row_block)
        z = h[r0:r1] @ W.T
        logp_all, m, R, lz = _log_softmax_block(z)
        p = np.exp(logp_all)
        rows = np.arange(r1 - r0)
        out["logp"][r0:r1] = logp_all[rows, y[r0:r1]]
        out["entropy"][r0:r1] = -(p * logp_all).sum(axis=1)
        out["lse"][r0:r1] = m + lz
        out["m"][r0:r1] = m
        out["R"][r0:r1] = R
    return out


def forward(hidden_bf16, weight_bf16, targets, row_block: int = ROW_BLOCK):
    """Forward on bf16 inputs (torch bf16 tensors or uint16 bits), in float64."""
    return forward_f64(_as_f64(hidden_bf16), _as_f64(weight_bf16), targets, row_block)


# --------------------------------------------------------------------------
# vocabulary-slice partials and their algebra
# --------------------------------------------------------------------------

def slice_partials_f64(h: np.ndarray, W_slice: np.ndarray, y: np.ndarray, vocab_start: int,
                       row_block: int = ROW_BLOCK):
    """Partial statistics of one vocabulary slice [vocab_start, vocab_start+Vs).

    Returns float64 arrays (m, R, B, zy), each [T]:
      m  = max over the slice, R = sum over the slice without its held-out
      argmax of exp(z - m), B = sum over the slice of exp(z - m) (z - m),
      zy = z_{y} when y falls in the slice, else -inf.
    """
    h = np.asarray(h, dtype=np.float64)
    W_slice = np.asarray(W_slice, dtype=np.float64)
    y = _as_index(y)
    T = h.shape[0]
    Vs = W_slice.shape[0]
    m_o, R_o, B_o, zy_o = (np.empty(T) for _ in range(4))
    for r0 in range(0, T, row_block):
        r1 = min(T, r0 + row_block)
        z = h[r0:r1] @ W_slice.T
        m, vstar, R, d = _row_stats(z)
        B = (np.exp(d) * d).sum(axis=1)
        loc = y[r0:r1] - vocab_start
        inside = (loc >= 0) & (loc < Vs)
        zy = np.full(r1 - r0, -np.inf)
        idx = np.nonzero(inside)[0]
        zy[idx] = z[idx, loc[idx]]
        m_o[r0:r1], R_o[r0:r1], B_o[r0:r1], zy_o[r0:r1] = m, R, B, zy
    return m_o, R_o, B_o, zy_o


def slice_partials(hidden_bf16, weight_slice_bf16, targets, vocab_start: int,
                   row_block: int = ROW_BLOCK):
    return slice_partials_f64(_as_f64(hidden_bf16), _as_f64(weight_slice_bf16), targets,
                              vocab_start, row_block)


def merge_partials(p1, p2):
    """Merge two partials (m, R, B, zy) over disjoint vocabulary sets.

    The side with the larger max is the base (the left operand on a tie), d =
    m_other - m_base <= 0 and, since exp(z - m_other) = exp(d) exp(z - m_base):

        R = R_base + exp(d) (1 + R_other)
        B = B_base + exp(d) (B_other + (1 + R_other) d)
        zy = the finite one (each target lies in exactly one set)
    """
    m1, R1, B1, zy1 = (np.asarray(a, dtype=np.float64) for a in p1)
    m2, R2, B2, zy2 = (np.asarray(a, dtype=np.float64) for a in p2)
    left = m1 >= m2
    mb = np.where(left, m1, m2)
    mo = np.where(left, m2, m1)
    Rb = np.where(left, R1, R2)
    Ro = np.where(left, R2, R1)
    Bb = np.where(left, B1, B2)
    Bo = np.where(left, B2, B1)
    d = mo - mb
    with np.errstate(invalid="ignore"):
        ed = np.exp(d)
        R = Rb + ed * (1.0 + Ro)
        B = Bb + ed * (Bo + (1.0 + Ro) * d)
    # a side whose max is -inf (empty) contributes nothing
    empty = np.isneginf(mo)
    R = np.where(empty, Rb, R)
    B = np.where(empty, Bb, B)
    zy = np.maximum(zy1, zy2)
    return mb, R, B, zy


def finalize_partials(p):
    """logp, entropy, lse from a whole-vocabulary partial (m, R, B, zy).

    log-normaliser relative to m is log1p(R); log p_y = (zy - m) - log1p(R);
    entropy = -sum p log p = log1p(R) - B / (1 + R).
    """
    m, R, B, zy = (np.asarray(a, dtype=np.float64) for a in p)
    lz = np.log1p(R)
    return {"logp": (zy - m) - lz, "entropy": lz - B / (1.0 + R), "lse": m + lz}


# --------------------------------------------------------------------------
# backward
# --------------------------------------------------------------------------

def backward_f64(h: np.ndarray, W: np.ndarray, y: np.ndarray, dlogp: np.ndarray,
                 dentropy: np.ndarray | None = None, *, dh_rows=None, dw_rows=None,
                 vocab_range: tuple[int, int] | None = None, with_abs: bool = False,
                 row_block: int = ROW_BLOCK):
    """Gradients of sum_t (dlogp_t logp_t + dent_t entropy_t) in float64.

    h [T,H], W [V,H] full vocabulary (the softmax always spans all V rows).
    dh_rows: token rows for which dH is returned (default all).
    dw_rows: vocabulary rows (global ids) for which dW is returned (default:
             all rows of ``vocab_range``).
    vocab_range: (a, b) restricts the vocabulary *contribution*: dH is then
             sum_{a <= v < b} G[:, v] W[v] (one slice's share) and dW rows must
             lie in [a, b). Default: the whole vocabulary.
    with_abs: also return the sums of the absolute values of the terms of each
             returned element, dH_abs = |G| |W| and dW_abs = |G|^T |h| over the
             same rows and vocabulary range (the scale of the rounding error of
             any summation of those terms).
    Returns dict with dH [len(dh_rows), H], dW [len(dw_rows), H], dh_rows, dw_rows
    (and dH_abs, dW_abs of the same shapes with ``with_abs``).
    """
    h = np.asarray(h, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    y = _as_index(y)
    T, H = h.shape
    V = W.shape[0]
    a, b = (0, V) if vocab_range is None else vocab_range
    dlogp = np.asarray(dlogp, dtype=np.float64)
    dent = np.zeros(T) if dentropy is None else np.asarray(dentropy, dtype=np.float64)
    dh_rows = np.arange(T) if dh_rows is None else np.asarray(dh_rows, dtype=np.int64)
    dw_rows = np.arange(a, b) if dw_rows is None else np.asarray(dw_rows, dtype=np.int64)
    if dw_rows.size and (dw_rows.min() < a or dw_rows.max() >= b):
        raise ValueError("dw_rows must lie inside vocab_range")
    dh_pos = {int(r): i for i, r in enumerate(dh_rows)}
    dH = np.zeros((dh_rows.size, H))
    dW = np.zeros((dw_rows.size, H))
    dH_abs = np.zeros((dh_rows.size, H)) if with_abs else None
    dW_abs = np.zeros((dw_rows.size, H)) if with_abs else None
    Wr = W[a:b]
    Wr_abs = np.abs(Wr) if with_abs else None
    for r0 in range(0, T, row_block):
        r1 = min(T, r0 + row_block)
        z = h[r0:r1] @ W.T
        logp_all, _, _, _ = _log_softmax_block(z)
        p = np.exp(logp_all)
        ent = -(p * logp_all).sum(axis=1)
        onehot = np.zeros_like(p)
        onehot[np.arange(r1 - r0), y[r0:r1]] = 1.0
        G = dlogp[r0:r1, None] * (onehot - p) - dent[r0:r1, None] * p * (logp_all + ent[:, None])
        Gr = G[:, a:b]
        sel = [t for t in range(r0, r1) if t in dh_pos]
        if sel:
            loc = np.array(sel) - r0
            dH[[dh_pos[t] for t in sel]] = Gr[loc] @ Wr
            if with_abs:
                dH_abs[[dh_pos[t] for t in sel]] = np.abs(Gr[loc]) @ Wr_abs
        dW += G[:, dw_rows].T @ h[r0:r1]
        if with_abs:
            dW_abs += np.abs(G[:, dw_rows]).T @ np.abs(h[r0:r1])
    out = {"dH": dH, "dW": dW, "dh_rows": dh_rows, "dw_rows": dw_rows}
    if with_abs:
        out.update({"dH_abs": dH_abs, "dW_abs": dW_abs})
    return out


def backward(hidden_bf16, weight_bf16, targets, dlogp, dentropy=None, **kw):
    """Backward on bf16 inputs (decoded exactly), float64 arithmetic."""
    return backward_f64(_as_f64(hidden_bf16), _as_f64(weight_bf16), targets,
                        _as_f64(dlogp), None if dentropy is None else _as_f64(dentropy), **kw)
