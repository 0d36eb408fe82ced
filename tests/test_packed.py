"""GPU tests of the packed-weight streaming forward (the rollout path).

The packed layout is a byte rearrangement declared in include/rlk_linear.h;
the device pack is compared byte for byte with that declaration written out
in numpy. The forward over a packed weight must return the same bits as the
natural-layout forward (which is checked against the oracle elsewhere, and
once more here at the bench shape): the rollout engine and the trainer then
score a token identically, the property the pages' batch-invariance evidence
asks of the linear-logp route ("RL-Kernel evidence h100-cp-gradient.json",
validation.train_rollout_logprob).
"""

import numpy as np
import pytest
import torch

import rollout_rlk_linear_amd as rlk
import workloads as wl
from oracle import forward
from tests._util import bits_equal, check_entropy, check_logp, dev

pytestmark = pytest.mark.gpu


def slicing(V, vs0, vt):
    """(P, Vs): the virtual-slice split the header declares."""
    if vt % 4 == 0:
        q = vt // 4
        if vs0 % q == 0 and V % q == 0:
            p, first = V // q, vs0 // q
            if p in (1, 2, 4) and first % p == 0:
                return p, q
    return 1, V


def pack_reference(W: np.ndarray, vs0: int, vt: int) -> np.ndarray:
    V, H = W.shape
    P, Vs = slicing(V, vs0, vt)
    Us = -(-Vs // 128)
    i = np.arange(64)
    r = i // 4
    piece = ((i % 4) - (r // 2)) % 4   # slot i % 4 of row r holds this 16-byte piece
    rows = 16 * np.arange(8)[:, None] + r[None, :]          # [block, lane]
    out = np.zeros((P * Us, H // 32, 8, 64, 8), dtype=np.uint16)
    for p in range(P):
        for iu in range(Us):
            R = np.zeros((128, H), dtype=np.uint16)
            blk = W[p * Vs + 128 * iu: p * Vs + min(128 * iu + 128, Vs)]
            R[:blk.shape[0]] = blk
            R4 = R.reshape(128, H // 32, 4, 8).transpose(1, 0, 2, 3)  # [step, row, piece, 8]
            out[p * Us + iu] = R4[:, rows, np.broadcast_to(piece, rows.shape), :]
    return out.reshape(-1)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("H,V,vs0,vt", [
    (64, 1000, 0, 1000),      # 4 virtual slices of 250 rows: partial units
    (128, 1001, 0, 1001),     # no slicing: one slice of 1001 rows
    (64, 500, 500, 1000),     # second half of a 2-way split
    (64, 250, 750, 1000),     # last quarter of a 4-way split
    (192, 128, 0, 128),       # exactly one unit
])
def test_pack_layout(H, V, vs0, vt):
    c = wl.make_case("pack", 1, H, V, 21, rms=False)
    W = dev(c.weight)
    pw = rlk.pack_weight(W, vocab_start=vs0, vocab_total=vt)
    torch.cuda.synchronize()
    got = pw.data.cpu().numpy().view(np.uint16)
    ref = pack_reference(bf16_bits(c.weight), vs0, vt)
    assert got.shape == ref.shape
    assert np.array_equal(got, ref), f"{int((got != ref).sum())} elements differ"


@pytest.mark.parametrize("T", [1, 2, 5, 20, 32, 64, 65, 130])
@pytest.mark.parametrize("H,V", [(128, 4000), (64, 1001), (256, 4 * 2500 + 4)])
def test_fwd_packed_bitwise(T, H, V):
    c = wl.make_case(f"pk{V}", T, H, V, 22 + T, rms=False)
    h, W, y = dev(c.hidden), dev(c.weight), dev(c.targets)
    ref = rlk.fwd(h, W, y)
    got = rlk.fwd_packed(h, rlk.pack_weight(W), y)
    torch.cuda.synchronize()
    for k in ("logp", "entropy", "stats"):
        assert bits_equal(got[k], ref[k]), f"T={T} H={H} V={V}: {k} differs"


@pytest.mark.parametrize("tp", [2, 4])
def test_fwd_packed_tp_slices(tp):
    c = wl.make_case("pktp", 33, 64, 1024, 23, rms=False)
    h, W, y = dev(c.hidden), dev(c.weight), dev(c.targets)
    V = W.shape[0]
    Vs = V // tp
    full = rlk.fwd(h, W, y)
    parts = []
    for k in range(tp):
        Wk = W[k * Vs:(k + 1) * Vs].contiguous()
        nat = rlk.fwd(h, Wk, y, vocab_start=k * Vs, vocab_total=V)["stats"]
        pk = rlk.fwd_packed(h, rlk.pack_weight(Wk, vocab_start=k * Vs, vocab_total=V), y)["stats"]
        torch.cuda.synchronize()
        assert bits_equal(pk, nat), f"TP={tp} slice {k}"
        parts.append(pk)
    comb = rlk.combine(parts)
    torch.cuda.synchronize()
    for k in ("logp", "entropy", "stats"):
        assert bits_equal(comb[k], full[k]), f"TP={tp}: combined {k}"


def test_fwd_packed_qwen_shape_against_oracle():
    # the rollout shape of the bench: T = 4 rows over W of 151936 x 4096
    c = wl.qwen512()
    W = dev(c.weight)
    h, y, _ = wl.qwen_rows(4, 31)
    pw = rlk.pack_weight(W)
    got = rlk.fwd_packed(dev(h), pw, dev(y))
    nat = rlk.fwd(dev(h), W, dev(y))
    torch.cuda.synchronize()
    for k in ("logp", "entropy", "stats"):
        assert bits_equal(got[k], nat[k]), k
    ref = forward(h, c.weight, y)
    check_logp(got["logp"].cpu().numpy(), ref["logp"], "packed T=4 logp")
    check_entropy(got["entropy"].cpu().numpy(), ref["entropy"], "packed T=4 entropy")
    del pw, W


def test_fwd_packed_reuses_buffers_across_sizes():
    # a second call with fewer rows into the same outputs and workspace
    c = wl.make_case("pkre", 40, 128, 3000, 24, rms=False)
    h, W, y = dev(c.hidden), dev(c.weight), dev(c.targets)
    pw = rlk.pack_weight(W)
    out = {}
    rlk.fwd_packed(h, pw, y, out=out)
    a = {k: v.clone() for k, v in out.items() if isinstance(v, torch.Tensor) and not k.startswith("_")}
    small = rlk.fwd_packed(h[:7].contiguous(), pw, y[:7].contiguous(), out={"_ws_fwdp": out["_ws_fwdp"]})
    torch.cuda.synchronize()
    for k in ("logp", "entropy", "stats"):
        assert bits_equal(small[k], a[k][:7]), k


@pytest.mark.parametrize("T", [1, 20, 70])
def test_forward_ignores_stale_workspace(T):
    # every record the combine reads is written by the same call: a workspace
    # full of NaN bytes gives the same bits as a zeroed one, for the tile and
    # stream forwards over natural W and for the packed forward
    H, V = 128, 1100
    c = wl.make_case("stalef", T, H, V, 43 + T, rms=False)
    h, W, y = dev(c.hidden), dev(c.weight), dev(c.targets)
    pw = rlk.pack_weight(W)
    lib = rlk.load_library()
    calls = {"_ws_fwd": (lib.rlk_linear_logp_fwd_workspace_bytes(T, H, V),
                         lambda o: rlk.fwd(h, W, y, out=o)),
             "_ws_fwdp": (lib.rlk_linear_logp_fwd_packed_workspace_bytes(T, H, V),
                          lambda o: rlk.fwd_packed(h, pw, y, out=o))}
    res = {}
    for fill in (0x00, 0xFF):  # 0xFF bytes: every fp32 value a NaN
        for key, (nws, call) in calls.items():
            ws = torch.full((max(nws, 256),), fill, dtype=torch.uint8, device="cuda")
            o = call({key: ws})
            torch.cuda.synchronize()
            res[key, fill] = {k: o[k].clone() for k in ("logp", "entropy", "stats")}
    for key in calls:
        for k in ("logp", "entropy", "stats"):
            assert bits_equal(res[key, 0xFF][k], res[key, 0x00][k]), f"{key} {k} T={T}"
    assert bits_equal(res["_ws_fwdp", 0x00]["stats"], res["_ws_fwd", 0x00]["stats"])
