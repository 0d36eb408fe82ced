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
    gpu = np.asarray(gpu, dtype=np.float64)
    assert np.isfinite(gpu).all(), f"{what}: non-finite gradient"
    nref = np.linalg.norm(ref)
    err = np.linalg.norm(gpu - ref) / max(nref, 1e-300)
    assert err <= GRAD_REL, f"{what}: rel Frobenius error {err:.3e}"
    return err


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
