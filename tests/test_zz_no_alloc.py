"""GPU test of the allocation-free forward (``rlk_linear_logp_fwd_noalloc``).

Its records go to the library's static device scratch instead of a caller
workspace; the kernels are those of ``rlk_linear_logp_fwd``, so every output
must be bit-identical to that entry point's on the same inputs. Two calls in
a row (the second smaller, so it leaves the first call's records in the part
of the scratch it does not write), then the first again, each checked bit for
bit; a slice call; and the limit reported as RLK_ERR_SCRATCH_LIMIT.
"""

import pytest
import torch

import rollout_rlk_linear_amd as rlk
import workloads as wl
from tests._util import bits_equal, case_to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rlk.load_library()


def same(a, b, what):
    for k in ("logp", "entropy", "stats"):
        if a[k] is None:
            assert b[k] is None, f"{what}: {k}"
            continue
        assert bits_equal(a[k], b[k]), f"{what}: {k} differs from the workspace entry point"


def test_noalloc_matches_workspace_forward_two_calls():
    c = wl.qwen512()  # T = 512 at H = 4096, V = 151936: the tile path, 4.9 MB of records
    d = case_to_device(c)
    small = 20        # the streaming path, 0.4 MB of records
    hs, ys = d["hidden"][:small].contiguous(), d["targets"][:small].contiguous()
    ref_big = rlk.fwd(d["hidden"], d["weight"], d["targets"])
    ref_small = rlk.fwd(hs, d["weight"], ys)
    torch.cuda.synchronize()
    n0 = rlk.call_count(6)
    print("noalloc call 1: T=512 H=4096 V=151936", flush=True)
    o1 = rlk.fwd_noalloc(d["hidden"], d["weight"], d["targets"])
    torch.cuda.synchronize()
    same(o1, ref_big, "call 1 (T=512)")
    print("noalloc call 2: T=20", flush=True)
    o2 = rlk.fwd_noalloc(hs, d["weight"], ys)
    torch.cuda.synchronize()
    same(o2, ref_small, "call 2 (T=20)")
    print("noalloc call 3: T=512 again", flush=True)
    o3 = rlk.fwd_noalloc(d["hidden"], d["weight"], d["targets"])
    torch.cuda.synchronize()
    same(o3, ref_big, "call 3 (T=512 after T=20)")
    assert rlk.call_count(6) == n0 + 3


def test_noalloc_slice_call_matches():
    # one TP=4 slice of a small vocabulary: the per-slice record
    c = wl.make_case("noalloc_slice", 70, 256, 4 * 1000, seed=91, rms=True)
    d = case_to_device(c)
    a, b = 1000, 2000
    Ws = d["weight"][a:b].contiguous()
    ref = rlk.fwd(d["hidden"], Ws, d["targets"], vocab_start=a, vocab_total=c.V)
    o = rlk.fwd_noalloc(d["hidden"], Ws, d["targets"], vocab_start=a, vocab_total=c.V)
    torch.cuda.synchronize()
    same(o, ref, "slice 1 of 4")


def test_noalloc_rejects_records_beyond_the_scratch():
    T, H, V = 879, 64, 151936
    h = torch.zeros(T, H, dtype=torch.bfloat16, device="cuda")
    W = torch.zeros(V, H, dtype=torch.bfloat16, device="cuda")
    y = torch.zeros(T, dtype=torch.int32, device="cuda")
    with pytest.raises(rlk.RlkError) as e:
        rlk.fwd_noalloc(h, W, y)
    assert e.value.status == 6
