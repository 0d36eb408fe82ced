"""GPU tensor-parallel-degree invariance of the forward and the backward (no
oracle applies: the GPU against itself).

The pages' strongest evidence for the linear-logp route is layout invariance:
the same log-probs, bit for bit, whatever the parallel layout of the actor
("RL-Kernel evidence h100-cp-gradient.json", the TP2/CP4 and TP4/CP2 runs;
the VIME page's actor runs at TP=4). With vocab_total a multiple of 4 the
library reduces 4 virtual vocabulary slices on their own and merges them by a
fixed tree, so a whole-vocabulary call (TP=1), two half-vocabulary calls
(TP=2) and four quarter calls (TP=4), each followed by the device combine,
must give identical logp, entropy and statistics bits. Values are checked
against the oracle elsewhere; here only equality matters. A split that does
not follow the virtual slices (3 pieces) still gives the right values, which
is checked against the full call within the tolerances.

The backward follows the same slices: dH splits start at each virtual slice's
first row and are sized by the slice, the slices' fp32 contributions add by
the same tree before the bf16 rounding, and rlk_linear_logp_dh_merge adds the
fp32 results of slice calls by that tree. So the merged dH of the TP = 2 and
TP = 4 slice calls has the bits of the whole-vocabulary call's dH (bf16 and
fp32), and every dW row of a slice call has the bits of the same row of the
whole-vocabulary call (the pages' gradient norms and parameter hashes are
equal across the TP2/CP4 and TP4/CP2 layouts: gradient_norm_comparisons,
all_parameter_hash_comparisons).
"""

import numpy as np
import pytest
import torch

import rollout_rlk_linear_amd as rlk
import workloads as wl
from tests._util import LOGP_ABS, ENT_REL, bits_equal, dev

pytestmark = pytest.mark.gpu


def tp_calls(h, W, y, tp):
    V = W.shape[0]
    Vs = V // tp
    parts = [rlk.fwd(h, W[k * Vs:(k + 1) * Vs].contiguous(), y, vocab_start=k * Vs,
                     vocab_total=V)["stats"] for k in range(tp)]
    return parts, rlk.combine(parts)


def check_tp(h, W, y, what):
    full = rlk.fwd(h, W, y)
    for tp in (1, 2, 4):
        parts, comb = tp_calls(h, W, y, tp)
        torch.cuda.synchronize()
        for k in ("logp", "entropy", "stats"):
            assert bits_equal(comb[k], full[k]), f"{what}: TP={tp} {k} differs from TP=1"
        if tp == 4:
            # the host combine uses the same tree with the host's exp/log1p
            lh, eh, sh = rlk.combine_host(parts)
            np.testing.assert_allclose(lh.numpy(), full["logp"].cpu().numpy(), rtol=0, atol=1e-5)
            np.testing.assert_allclose(eh.numpy(), full["entropy"].cpu().numpy(), rtol=1e-5)
    return full


@pytest.mark.parametrize("T,H,V,seed", [(70, 128, 4000, 9), (33, 64, 1024, 10), (300, 256, 4 * 2500, 11)])
def test_tp_degree_bitwise_small(T, H, V, seed):
    c = wl.make_case(f"tp{V}", T, H, V, seed, rms=False)
    check_tp(dev(c.hidden), dev(c.weight), dev(c.targets), f"T={T} H={H} V={V}")


def test_tp_degree_bitwise_long_response():
    # the 7168-token long-response case over the full 151,936-row vocabulary
    c = wl.slice7168()
    h, W, y = dev(c.hidden), dev(c.weight), dev(c.targets)
    full = check_tp(h, W, y, "T=7168 V=151936")
    # a split that does not follow the virtual slices: correct values, no bit promise
    V = W.shape[0]
    cuts = [0, 50000, 100032, V]
    parts = [rlk.fwd(h, W[a:b].contiguous(), y, vocab_start=a, vocab_total=V)["stats"]
             for a, b in zip(cuts[:-1], cuts[1:])]
    comb = rlk.combine(parts)
    torch.cuda.synchronize()
    dl = (comb["logp"] - full["logp"]).abs().max().item()
    de = ((comb["entropy"] - full["entropy"]).abs() / full["entropy"].abs()).max().item()
    # both sides are within the tolerances of the exact values, so within twice of each other
    assert dl <= 2 * LOGP_ABS and de <= 2 * ENT_REL, (dl, de)
    del W


def dev_equal(a, b):
    """Bitwise equality on the device (large tensors stay there)."""
    if a.shape != b.shape or a.dtype != b.dtype:
        return False
    iv = torch.int32 if a.dtype == torch.float32 else torch.int16
    return bool(torch.equal(a.contiguous().view(iv), b.contiguous().view(iv)))


def check_tp_backward(h, W, y, dl, de, what):
    V = W.shape[0]
    full = rlk.fwd(h, W, y)
    dh1, dw1 = rlk.bwd(h, W, y, full["stats"], dl, de)
    dh1f, _ = rlk.bwd(h, W, y, full["stats"], dl, de, dhidden_f32=True, want_dweight=False)
    torch.cuda.synchronize()
    for tp in (1, 2, 4):
        Vs = V // tp
        dhs = []
        for k in range(tp):
            print(f"{what}: TP={tp} slice {k} backward", flush=True)
            dh, dw = rlk.bwd(h, W[k * Vs:(k + 1) * Vs].contiguous(), y, full["stats"], dl, de,
                             vocab_start=k * Vs, vocab_total=V, dhidden_f32=True)
            torch.cuda.synchronize()
            assert dev_equal(dw, dw1[k * Vs:(k + 1) * Vs]), f"{what}: TP={tp} slice {k} dW rows differ"
            dhs.append(dh)
            del dw
        merged = rlk.dh_merge(dhs)
        merged_f = rlk.dh_merge(dhs, f32=True)
        torch.cuda.synchronize()
        assert dev_equal(merged, dh1), f"{what}: TP={tp} merged dH (bf16) differs from TP=1"
        assert dev_equal(merged_f, dh1f), f"{what}: TP={tp} merged dH (fp32) differs from TP=1"
        del dhs, merged, merged_f


@pytest.mark.parametrize("T,H,V,seed", [(70, 128, 4000, 9), (33, 64, 1024, 10),
                                        (300, 256, 4 * 2500, 11), (5, 192, 4 * 1100, 12)])
def test_tp_degree_backward_bitwise_small(T, H, V, seed):
    c = wl.make_case(f"tpb{V}", T, H, V, seed, rms=True)
    c.weight = wl.to_bf16(c.weight.float() * 20)  # logits of spread ~ 1.3
    check_tp_backward(dev(c.hidden), dev(c.weight), dev(c.targets), dev(c.dlogp),
                      dev(c.dentropy), f"T={T} H={H} V={V}")


def test_tp_degree_backward_bitwise_long_response():
    # the 7168-token long-response case over the full 151,936-row vocabulary,
    # with an entropy gradient as well
    c = wl.slice7168()
    de = torch.randn(c.T, generator=torch.Generator().manual_seed(16), dtype=torch.float32)
    check_tp_backward(dev(c.hidden), dev(c.weight), dev(c.targets), dev(c.dlogp), dev(de),
                      "T=7168 V=151936")
