"""GPU bitwise batch invariance (no oracle applies: the GPU against itself).

The pages' acceptance form for the linear-logp route is zero bitwise
mismatches and max |diff| = 0 between the trainer's large packed batches and
the rollout engine's CUDA-graph batches of 1 to 4 ("RL-Kernel evidence
h100-cp-gradient.json", validation.train_rollout_logprob and
validation.cudagraph.expected_capture_sizes). Here a fixed pool of 64
Qwen3-8B-shaped rows (H = 4096, V = 151936) is scored in batches of 1, 2, 3,
4, 24 and 64, under 3 row permutations, embedded in a batch of 512 other rows,
and repeated, and scored through the packed-weight rollout path in batches
of 1 to 4, 24 and 64; every row's logp, entropy and statistics record must be
bit-identical across all of them. The same holds for each row of dhidden,
also inside 200- and 768-row batches (the two load policies of W), and for
calls issued on two streams at once.
"""

import pytest
import torch

import rollout_rlk_linear_amd as rlk
import workloads as wl
from tests._util import bits_equal, dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    W = dev(wl.qwen512().weight)
    pool = wl.pool64()
    _, _, dlogp = wl.qwen_rows(64, 2)
    return {"W": W, "h": dev(pool["hidden"]), "y": dev(pool["targets"]), "dlogp": dev(dlogp),
            "pool": pool}


def score(W, h, y):
    o = rlk.fwd(h, W, y)
    return torch.stack([o["logp"], o["entropy"]], dim=1), o["stats"]


def batched(W, h, y, bs):
    outs, stats = [], []
    for r0 in range(0, h.shape[0], bs):
        a, s = score(W, h[r0:r0 + bs].contiguous(), y[r0:r0 + bs].contiguous())
        outs.append(a)
        stats.append(s)
    return torch.cat(outs), torch.cat(stats)


def mismatch(a, b):
    return int((a.contiguous().view(torch.int32) != b.contiguous().view(torch.int32)).sum())


def test_batch_sizes_bitwise(setup):
    W, h, y = setup["W"], setup["h"], setup["y"]
    ref, ref_st = score(W, h, y)
    torch.cuda.synchronize()
    assert torch.isfinite(ref).all()
    for bs in (1, 2, 3, 4, 24, 64):
        for rep in range(3):
            got, st = batched(W, h, y, bs)
            torch.cuda.synchronize()
            assert mismatch(got, ref) == 0, f"batch {bs} repeat {rep}"
            assert mismatch(st, ref_st) == 0, f"stats, batch {bs} repeat {rep}"
            assert float((got - ref).abs().max()) == 0.0


def test_permutations_bitwise(setup):
    W, h, y = setup["W"], setup["h"], setup["y"]
    ref, ref_st = score(W, h, y)
    for perm in setup["pool"]["perms"]:
        p = perm.cuda()
        got, st = score(W, h[p].contiguous(), y[p].contiguous())
        inv = torch.argsort(p)
        torch.cuda.synchronize()
        assert mismatch(got[inv], ref) == 0
        assert mismatch(st[inv], ref_st) == 0


def test_composition_bitwise(setup):
    W, h, y = setup["W"], setup["h"], setup["y"]
    ref, ref_st = score(W, h, y)
    emb = setup["pool"]["embed"]
    pos = emb["positions"].cuda()
    for rep in range(2):
        got, st = score(W, dev(emb["hidden"]), dev(emb["targets"]))
        torch.cuda.synchronize()
        assert mismatch(got[pos], ref) == 0
        assert mismatch(st[pos], ref_st) == 0


def test_rollout_packed_batches_match_training_batch(setup):
    # the rollout engine's path (packed W, decode batches of 1 to 4, 24 and 64)
    # against the trainer's: the pool's rows inside a 512-row batch
    W, h, y = setup["W"], setup["h"], setup["y"]
    emb = setup["pool"]["embed"]
    pos = emb["positions"].cuda()
    train, train_st = score(W, dev(emb["hidden"]), dev(emb["targets"]))
    pw = rlk.pack_weight(W)
    for bs in (1, 2, 3, 4, 24, 64):
        outs, stats = [], []
        for r0 in range(0, 64, bs):
            o = rlk.fwd_packed(h[r0:r0 + bs].contiguous(), pw, y[r0:r0 + bs].contiguous())
            outs.append(torch.stack([o["logp"], o["entropy"]], dim=1))
            stats.append(o["stats"])
        torch.cuda.synchronize()
        assert mismatch(torch.cat(outs), train[pos]) == 0, f"rollout batch {bs}"
        assert mismatch(torch.cat(stats), train_st[pos]) == 0, f"rollout stats, batch {bs}"
    del pw


def test_dhidden_rows_bitwise(setup):
    W, h, y, dl = setup["W"], setup["h"], setup["y"], setup["dlogp"]
    _, st = score(W, h, y)
    ref, _ = rlk.bwd(h, W, y, st, dl, None, want_dweight=False)
    torch.cuda.synchronize()
    # single rows and a batch of 4 at various positions
    for r in (0, 17, 63):
        got, _ = rlk.bwd(h[r:r + 1].contiguous(), W, y[r:r + 1].contiguous(), st[r:r + 1].contiguous(),
                         dl[r:r + 1].contiguous(), None, want_dweight=False)
        torch.cuda.synchronize()
        assert bits_equal(got[0], ref[r]), f"row {r}"
    got, _ = rlk.bwd(h[8:12].contiguous(), W, y[8:12].contiguous(), st[8:12].contiguous(),
                     dl[8:12].contiguous(), None, want_dweight=False)
    torch.cuda.synchronize()
    assert bits_equal(got, ref[8:12])
    # embedded in the 512-row batch (large-tile path)
    emb = setup["pool"]["embed"]
    he, ye = dev(emb["hidden"]), dev(emb["targets"])
    _, ste = score(W, he, ye)
    dle = torch.zeros(512, device="cuda")
    pos = emb["positions"].cuda()
    dle[pos] = dl
    got, _ = rlk.bwd(he, W, ye, ste, dle, None, want_dweight=False)
    torch.cuda.synchronize()
    assert bits_equal(got[pos], ref)


@pytest.mark.parametrize("T", [200, 768])
def test_rows_bitwise_across_cache_policies(setup, T):
    """The load policy of W changes with the batch. The forward's tile kernel
    reads W non-temporally when the batch is one T-tile (65 to 256 rows) and
    with the default policy for more; the recompute of G reads it
    non-temporally while the batch's bf16 G fits in 192 MiB (up to 640 rows
    at V = 151936) and with the default policy above that. A cache hint must
    not change a bit: the pool's rows inside a 200-row batch (both hints on)
    and inside a 768-row batch (both off, G of 223 MiB) give the records and
    dhidden rows that the 64-row batch gives on the small-batch kernels."""
    W, h, y, dl = setup["W"], setup["h"], setup["y"], setup["dlogp"]
    ref, ref_st = score(W, h, y)
    ref_dh, _ = rlk.bwd(h, W, y, ref_st, dl, None, want_dweight=False)
    g_fits = (T + 31) // 32 * 32 * W.shape[0] * 2 <= (192 << 20)
    one_tile = 64 < T <= 256
    assert (g_fits, one_tile) == ((True, True) if T == 200 else (False, False))
    big_h, big_y, _ = wl.qwen_rows(T, 11)
    pos = torch.randperm(T, generator=torch.Generator().manual_seed(12))[:64]
    big_h[pos] = setup["pool"]["hidden"]
    big_y[pos] = setup["pool"]["targets"]
    big_h, big_y, pos = dev(big_h), dev(big_y), pos.cuda()
    got, st = score(W, big_h, big_y)
    dlb = torch.zeros(T, device="cuda")
    dlb[pos] = dl
    dh, _ = rlk.bwd(big_h, W, big_y, st, dlb, None, want_dweight=False)
    torch.cuda.synchronize()
    assert mismatch(got[pos], ref) == 0
    assert mismatch(st[pos], ref_st) == 0
    assert bits_equal(dh[pos], ref_dh)


def test_concurrent_streams_bitwise(setup):
    """Two forward + backward calls issued on two streams at once, each with
    its own workspace, give the bits the same calls give one after the
    other: the library keeps no state between calls that the kernels of
    one call could see from another."""
    W, h, y, dl = setup["W"], setup["h"], setup["y"], setup["dlogp"]
    emb = setup["pool"]["embed"]
    he, ye = dev(emb["hidden"]), dev(emb["targets"])
    dle = torch.randn(he.shape[0], generator=torch.Generator().manual_seed(13)).cuda()

    def run(hh, yy, dd):
        o = rlk.fwd(hh, W, yy)
        dh, dw = rlk.bwd(hh, W, yy, o["stats"], dd, None)
        return o["stats"], dh, dw

    serial = [run(h, y, dl), run(he, ye, dle)]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]  # default priority
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(streams[0]):
        a = run(h, y, dl)
    with torch.cuda.stream(streams[1]):
        b = run(he, ye, dle)
    torch.cuda.synchronize()
    for got, ref in zip((a, b), serial):
        for g, r in zip(got, ref):
            assert bits_equal(g, r)


def test_dweight_repeat_deterministic(setup):
    W, h, y, dl = setup["W"], setup["h"], setup["y"], setup["dlogp"]
    _, st = score(W, h, y)
    dh1, dw1 = rlk.bwd(h, W, y, st, dl, None)
    dh2, dw2 = rlk.bwd(h, W, y, st, dl, None)
    torch.cuda.synchronize()
    assert bits_equal(dw1, dw2) and bits_equal(dh1, dh2)


@pytest.mark.parametrize("T,H,V", [(65, 64, 1001), (130, 64, 1001), (300, 192, 4000),
                                   (257, 4096, 151936)])
def test_tile_forward_repeats_bitwise(T, H, V):
    """Repeated calls of the large-batch forward give the same bits every time,
    and the same bits as the streaming path over the packed weight, at shapes
    where the mainloop has one or three k-step pairs (H = 64, 192) and the
    last vocabulary group is partial (V = 1001, 4000), and at the full LM-head
    width; streaming calls between the repeats vary the timing."""
    c = wl.make_case(f"rep{V}", T, H, V, 31 + T, rms=False)
    h, W, y = dev(c.hidden), dev(c.weight), dev(c.targets)
    pw = rlk.pack_weight(W)
    first = rlk.fwd(h, W, y)["stats"].clone()
    streamed = rlk.fwd_packed(h, pw, y)["stats"]
    torch.cuda.synchronize()
    assert bits_equal(first, streamed), f"T={T} H={H} V={V}: tile and stream records differ"
    reps = 40 if H < 4096 else 8
    out = {}
    for k in range(reps):
        got = rlk.fwd(h, W, y, out=out)["stats"]
        if k % 2:
            rlk.fwd_packed(h, pw, y)
        torch.cuda.synchronize()
        bad = int((got.view(torch.int32) != first.view(torch.int32)).any(dim=1).sum())
        assert bad == 0, f"T={T} H={H} V={V}: repeat {k} differs in {bad} rows"
