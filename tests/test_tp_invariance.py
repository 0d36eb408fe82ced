"""GPU tensor-parallel-degree invariance of the forward (no oracle applies:
the GPU against itself).

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
