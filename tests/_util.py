"""Shared helpers for the GPU tests: tolerances, comparisons, device copies."""

import numpy as np
import torch

# Tolerances of the operator (per row for logp and entropy, norm-wise for gradients).
LOGP_ABS = 1e-3
ENT_REL = 1e-3
GRAD_REL = 5e-3


def dev(x):
    return None if x is None else x.to("cuda").contiguous()


def case_to_device(c):
    return {"hidden": dev(c.hidden), "weight": dev(c.weight), "targets": dev(c.targets),
            "dlogp": dev(c.dlogp), "dentropy": dev(c.dentropy)}


def check_logp(gpu, ref, what=""):
    gpu = np.asarray(gpu, dtype=np.float64)
    d = np.abs(gpu - ref)
    assert np.isfinite(gpu).all(), f"{what}: non-finite logp"
    assert d.max() <= LOGP_ABS, f"{what}: max |dlogp| = {d.max():.3e} at row {d.argmax()}"
    return d.max()


def check_entropy(gpu, ref, what=""):
    gpu = np.asarray(gpu, dtype=np.float64)
    rel = np.abs(gpu - ref) / np.maximum(np.abs(ref), 1e-30)
    assert np.isfinite(gpu).all(), f"{what}: non-finite entropy"
    assert rel.max() <= ENT_REL, (f"{what}: max rel dentropy = {rel.max():.3e} at row {rel.argmax()}"
                                  f" (gpu {gpu[rel.argmax()]:.6e}, ref {ref[rel.argmax()]:.6e})")
    return rel.max()


def check_grad(gpu, ref, what=""):
    """Whole-tensor relative Frobenius error <= GRAD_REL, and the same bound
    for every row on its own (a localised error cannot hide in the norm)."""
    gpu = np.asarray(gpu, dtype=np.float64)
    assert np.isfinite(gpu).all(), f"{what}: non-finite gradient"
    nref = np.linalg.norm(ref)
    err = np.linalg.norm(gpu - ref) / max(nref, 1e-300)
    assert err <= GRAD_REL, f"{what}: rel Frobenius error {err:.3e}"
    check_grad_rows(gpu, ref, what)
    return err


def check_grad_rows(gpu, ref, what=""):
    """Per row: ||gpu_row - ref_row|| <= GRAD_REL ||ref_row||; a row whose
    reference is exactly zero must come out exactly zero."""
    gpu = np.asarray(gpu, dtype=np.float64).reshape(len(ref), -1)
    ref = np.asarray(ref, dtype=np.float64).reshape(len(ref), -1)
    dn = np.linalg.norm(gpu - ref, axis=1)
    rn = np.linalg.norm(ref, axis=1)
    zero = rn == 0
    assert (dn[zero] == 0).all(), f"{what}: rows {np.nonzero(zero & (dn > 0))[0][:8]} should be 0"
    rel = dn[~zero] / rn[~zero]
    if rel.size:
        i = int(rel.argmax())
        assert rel.max() <= GRAD_REL, (f"{what}: row {np.nonzero(~zero)[0][i]} rel error "
                                       f"{rel.max():.3e} > {GRAD_REL}")
    return float(rel.max()) if rel.size else 0.0


# Element bound of a gradient against float64. Every element is a sum of
# products G[t, v] x (W or hidden) with the logit gradient G rounded to bf16
# (round to nearest even: relative error at most 2^-8) after an fp32
# computation from the fp32 logits (allowance 2^-10 relative, some twenty
# times what the logits' accumulation and the exponentials contribute at
# these scales), summed by an fp32 chain of n_terms additions
# (n_terms 2^-24 of the sum of |terms|), and the output itself rounded (half a
# bf16 ulp, or 2^-24 relative for fp32).
G_REL = 2.0 ** -8 + 2.0 ** -10


def check_grad_elements(gpu, ref, abs_terms, n_terms, what=""):
    """|gpu - ref| <= out_rounding + (G_REL + n_terms 2^-24) abs_terms per element;
    abs_terms = sum of |terms| of the element (the oracle's dH_abs / dW_abs)."""
    if isinstance(gpu, torch.Tensor):
        bf16 = gpu.dtype == torch.bfloat16
        gpu = f64(gpu)
    else:
        bf16 = False
    gpu = np.asarray(gpu, dtype=np.float64)
    if bf16:
        out_round = 0.5 * np.spacing(np.abs(gpu).astype(np.float32)).astype(np.float64) * 2.0 ** 16
    else:
        out_round = 2.0 ** -24 * np.abs(gpu)
    bound = out_round + (G_REL + n_terms * 2.0 ** -24) * abs_terms
    excess = np.abs(gpu - ref) - bound
    assert (excess <= 0).all(), (f"{what}: {(excess > 0).sum()} elements beyond the bound, "
                                 f"worst at {np.unravel_index(excess.argmax(), excess.shape)} "
                                 f"by {excess.max():.3e}")
    return float((np.abs(gpu - ref) / np.maximum(bound, 1e-300)).max())


def f64(t):
    if t.dtype == torch.bfloat16:
        return t.float().cpu().double().numpy()
    return t.cpu().double().numpy()


def bits_equal(a, b):
    """Bitwise equality of two float tensors (NaNs compare by pattern)."""
    a = a.contiguous().cpu()
    b = b.contiguous().cpu()
    if a.shape != b.shape:
        return False
    if a.dtype == torch.float32:
        return torch.equal(a.view(torch.int32), b.view(torch.int32))
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a, b)
