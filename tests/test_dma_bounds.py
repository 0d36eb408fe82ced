"""Address model of the LDS-DMA operand staging (CPU only, no GPU).

The mainloops in ``rlk_device.h`` and the small-batch stream in
``rlk_kernels.hip`` fetch operands with gfx950 raw buffer loads
(``buffer_load_dwordx4 ... offen lds``): lane i fetches the 16 bytes at
base + soffset + voffset, and the hardware range check compares the vector
offset alone with the descriptor's num_records (a load whose voffset is at or
past it returns zeros and touches no memory; the scalar offset is outside the
check). These tests recompute, from the same formulas the kernels use, the
(voffset, soffset, num_records) triple of every lane, wave, DMA block and
stage, and check two things for ragged operands:

* every byte that is fetched lies inside the caller's operand (rows at or past
  the valid count are never read), and
* every 16-byte piece of every valid row inside the k range is fetched
  exactly once per use (the staging loses nothing).

A planted control reproduces the former form of ``AsyncGemmP`` (32-row block
offsets in the scalar offset) and checks that the model flags its reads past
the operand.
"""

import numpy as np
import pytest

LANES = np.arange(64)


class Fetches:
    """Fetched 16-byte pieces of one operand, as byte offsets from its base."""

    def __init__(self):
        self.addrs = []

    def issue(self, voff, soff, nrec, base=0):
        voff = np.broadcast_to(np.asarray(voff, dtype=np.int64), LANES.shape)
        ok = voff < nrec
        self.addrs.append(base + soff + voff[ok])

    def all(self):
        return np.concatenate(self.addrs) if self.addrs else np.zeros(0, np.int64)


def check_k_contiguous(f, rows, ld, k_begin, k_end, what):
    """Fetched pieces of a K-contiguous operand (element (r, k) at r*ld + k)."""
    a = f.all()
    assert a.size == 0 or (a.min() >= 0 and (a + 16).max() <= rows * ld * 2), (
        f"{what}: fetch outside rows [0, {rows}) (max end {(a + 16).max()}, "
        f"extent {rows * ld * 2})")
    want = (np.arange(rows)[:, None] * ld * 2 + np.arange(2 * k_begin, 2 * k_end, 16)[None, :]).ravel()
    got, cnt = np.unique(a, return_counts=True)
    assert np.array_equal(got, np.sort(want)), f"{what}: fetched pieces differ from the valid ones"
    assert (cnt == 1).all(), f"{what}: a piece fetched twice"


def check_k_major(f, k_valid, n_valid, ld, what):
    """Fetched pieces of a K-major operand (element (k, n) at k*ld + n): the
    extent ends at column n_valid of row k_valid - 1."""
    a = f.all()
    end = ((k_valid - 1) * ld + n_valid) * 2 if k_valid > 0 else 0
    assert a.size == 0 or (a.min() >= 0 and (a + 16).max() <= end), (
        f"{what}: fetch outside the operand (max end {(a + 16).max()}, extent {end})")


# ----------------------------------------------------------- AsyncGemmP --

def model_gemm_p(BM, BN, lda, ldb, a_rows, b_rows, k_begin, k_end, rows_in_scalar=False):
    NW = 4
    NI_A, NI_B = BM // 8, BN // 8
    NB = (NI_A + NI_B) // NW
    NB_A = NI_A // NW
    ar, br = min(max(a_rows, 0), BM), min(max(b_rows, 0), BN)
    fa, fb = Fetches(), Fetches()
    for wave in range(NW):
        row0 = 8 * wave + (LANES >> 3)
        piece = ((LANES & 7) - (row0 & 15)) & 7
        voffA = row0 * lda * 2 + 16 * piece
        voffB = row0 * ldb * 2 + 16 * piece
        for p in range((k_end - k_begin) // 64):
            koff = (k_begin + 64 * p) * 2
            for ii in range(NB):
                if ii < NB_A:
                    if rows_in_scalar:
                        fa.issue(voffA, koff + ii * 64 * lda, ar * lda * 2)
                    else:
                        fa.issue(voffA + ii * 64 * lda, koff, ar * lda * 2)
                else:
                    jj = ii - NB_A
                    if rows_in_scalar:
                        fb.issue(voffB, koff + jj * 64 * ldb, br * ldb * 2)
                    else:
                        fb.issue(voffB + jj * 64 * ldb, koff, br * ldb * 2)
    return fa, fb


# (BM, BN): fwd_tile and the large-batch recompute, the small-batch
# recompute, the LoRA forward (wide and narrow tiles)
GEMM_P = [(256, 256), (32, 128), (64, 128), (64, 32)]


@pytest.mark.parametrize("BM,BN", GEMM_P)
@pytest.mark.parametrize("a_rows,b_rows", [(1, 1), (5, 33), (70, 200), (31, 129), (256, 256),
                                           (300, 1000), (64, 128)])
@pytest.mark.parametrize("H", [64, 192])
def test_gemm_p_reads_only_valid_rows(BM, BN, a_rows, b_rows, H):
    fa, fb = model_gemm_p(BM, BN, H, H, a_rows, b_rows, 0, H)
    check_k_contiguous(fa, min(a_rows, BM), H, 0, H, f"A {BM}x{BN} rows={a_rows}")
    check_k_contiguous(fb, min(b_rows, BN), H, 0, H, f"B {BM}x{BN} rows={b_rows}")


@pytest.mark.parametrize("k_begin,k_end", [(0, 128), (128, 256), (64, 192)])
def test_gemm_p_k_split_reads_only_its_range(k_begin, k_end):
    # the LoRA forward's split contraction: k over [k_begin, k_end) of H = 256
    fa, fb = model_gemm_p(64, 32, 256, 256, 33, 20, k_begin, k_end)
    check_k_contiguous(fa, 33, 256, k_begin, k_end, "A split")
    check_k_contiguous(fb, 20, 256, k_begin, k_end, "B split")


def test_gemm_p_planted_scalar_row_offsets_are_caught():
    # the former placement: rows 32 ii of a block in the unchecked scalar offset
    fa, _ = model_gemm_p(256, 256, 128, 128, 70, 256, 0, 128, rows_in_scalar=True)
    with pytest.raises(AssertionError, match="outside"):
        check_k_contiguous(fa, 70, 128, 0, 128, "planted")


# ---------------------------------------------------------- AsyncGemmKN --

def bswz(k):
    return 2 * (k & 3) + 8 * ((k >> 3) & 1)


def model_gemm_kn(BM, BN, lda, a_rows, ldb, kb_valid, nb_valid, k_begin, k_end, NST=4):
    NW = 4
    NI_A, NI_B = BM * 64 // 1024, 32 * BN * 2 // 1024
    NI = NI_A + NI_B
    # the ring is padded: NST - 1 stages past the last one go out through
    # empty resources (A's with no records, since its k offset is in the
    # scalar offset; B's rows clamp to none)
    PPR = BN // 8
    RPB = 64 // PPR
    ar = min(max(a_rows, 0), BM)
    fa, fb = Fetches(), Fetches()
    drow = LANES >> 2
    dpiece = ((LANES & 3) - (drow >> 1)) & 3
    brow, bslot = LANES // PPR, LANES % PPR
    nsteps = (k_end - k_begin) // 32
    for wave in range(NW):
        for s in range(nsteps + NST - 1):
            k0 = k_begin + 32 * s
            brows = min(max(kb_valid - k0, 0), 32)
            bbytes = ((brows - 1) * ldb + nb_valid) * 2 if brows > 0 else 0
            for ii in range((NI + NW - 1) // NW):
                j = wave + NW * ii
                if j >= NI:
                    continue
                if j < NI_A:
                    fa.issue((16 * j + drow) * lda * 2 + 16 * dpiece, k0 * 2,
                             ar * lda * 2 if s < nsteps else 0)
                else:
                    k = RPB * (j - NI_A) + brow
                    fb.issue(k * ldb * 2 + 16 * (bslot ^ bswz(k)), 0, bbytes, base=k0 * ldb * 2)
    return fa, fb


# (BM, BN): dH at large and small batches, LoRA dx
@pytest.mark.parametrize("BM,BN", [(256, 256), (32, 128), (64, 128)])
@pytest.mark.parametrize("a_rows,kb_valid,H,h0", [(70, 300, 320, 256), (1, 33, 128, 0),
                                                  (256, 1000, 512, 256), (40, 64, 64, 0),
                                                  (300, 77, 320, 0)])
def test_gemm_kn_reads_inside_operands(BM, BN, a_rows, kb_valid, H, h0):
    if h0 >= H:
        pytest.skip("no such h-tile")
    ldg = ((kb_valid + 31) // 32) * 32 + 64   # G rows: the split columns and some more
    k_end = (kb_valid + 31) // 32 * 32
    nb_valid = min(BN, H - h0)
    fa, fb = model_gemm_kn(BM, BN, ldg, a_rows, H, kb_valid, nb_valid, 0, k_end)
    check_k_contiguous(fa, min(a_rows, BM), ldg, 0, k_end, f"KN A {BM}x{BN}")
    check_k_major(fb, kb_valid, nb_valid, H, f"KN B {BM}x{BN}")


# ---------------------------------------------------------- AsyncGemmKK --

def model_gemm_kk(BM, BN, lda, ka_valid, na_valid, ldb, kb_valid, nb_valid, k_begin, k_end,
                  pad=False, NST=3):
    NW = 4
    PPR_A, PPR_B = BM // 8, BN // 8
    RPB_A, RPB_B = 64 // PPR_A, 64 // PPR_B
    NI_A, NI_B = 32 * BM * 2 // 1024, 32 * BN * 2 // 1024
    NB = (NI_A + NI_B) // NW
    fa, fb = Fetches(), Fetches()

    def stage(ld, k0, kv, nv):
        rows = min(max(kv - k0, 0), 32)
        return ((rows - 1) * ld + nv) * 2 if rows > 0 else 0

    nsteps = (k_end - k_begin) // 32
    for wave in range(NW):
        # padded: NST - 1 stages past the last, whose rows clamp to none
        for s in range(nsteps + (NST - 1 if pad else 0)):
            k0 = k_begin + 32 * s
            for ii in range(NB):
                j = wave + NW * ii
                if ii < NI_A // NW:
                    k = RPB_A * j + LANES // PPR_A
                    fa.issue(k * lda * 2 + 16 * ((LANES % PPR_A) ^ bswz(k)), 0,
                             stage(lda, k0, ka_valid, na_valid), base=k0 * lda * 2)
                else:
                    k = RPB_B * (j - NI_A) + LANES // PPR_B
                    fb.issue(k * ldb * 2 + 16 * ((LANES % PPR_B) ^ bswz(k)), 0,
                             stage(ldb, k0, kb_valid, nb_valid), base=k0 * ldb * 2)
    return fa, fb


@pytest.mark.parametrize("T,H,h0", [(1, 128, 0), (70, 320, 256), (512, 256, 128), (33, 64, 0)])
def test_gemm_kk_reads_inside_operands(T, H, h0):
    # dW: A = G [t][v] (256 columns of a ldg-wide row), B = hidden [t][h]
    ldg = 1024
    Tp = (T + 31) // 32 * 32
    fa, fb = model_gemm_kk(256, 128, ldg, T, 256, H, T, min(128, H - h0), 0, Tp, pad=Tp > 64)
    check_k_major(fa, T, 256, ldg, "KK A (G)")
    check_k_major(fb, T, min(128, H - h0), H, "KK B (hidden)")


# ------------------------------------------------------ fwd_stream_kernel --

def model_stream(MI, KS, packed, T, H, vrows):
    """One unit of the streaming forward: hidden (T rows, or 16 MI) and a
    128-row unit of W (vrows valid rows; packed: the whole 128 H unit)."""
    NW = 4
    fa, fb = Fetches(), Fetches()
    nrecA = min(T, 16 * MI) * H * 2
    nrecB = 128 * H * 2 if packed else vrows * H * 2
    nsteps = H // (32 * KS)
    drow = LANES >> 2
    dpiece = ((LANES & 3) - (drow >> 1)) & 3
    prow_of = lambda wave: 8 * wave + (LANES >> 3)
    for wave in range(NW):
        prow = prow_of(wave)
        ppiece = ((LANES & 7) - prow) & 7
        for s in range(nsteps):
            if KS == 1:
                if wave < MI:
                    fa.issue((16 * wave + drow) * H * 2 + 16 * dpiece, 64 * s, nrecA)
                for w2 in (wave, wave + 4):
                    v = 1024 * w2 + 16 * LANES if packed else (16 * w2 + drow) * H * 2 + 16 * dpiece
                    fb.issue(v, (8192 if packed else 64) * s, nrecB)
            else:
                NA2 = 2 * MI
                nA2w = (NA2 - wave + 3) // 4 if wave < NA2 else 0
                for k in range(2):
                    if k < nA2w:
                        fa.issue((prow + 32 * k) * H * 2 + 16 * ppiece, 128 * s, nrecA)
                for k in range(4):
                    v = (1024 * (wave + 4 * k) + 16 * LANES if packed
                         else (prow + 32 * k) * H * 2 + 16 * ppiece)
                    fb.issue(v, (16384 if packed else 128) * s, nrecB)
    return fa, fb


# (MI, KS, T, vrows): the launcher runs MI 16-row blocks for T <= 16 MI rows
STREAM_CASES = [(mi, ks, t, vr)
                for mi, ks in [(1, 1), (2, 1), (4, 1), (1, 2), (2, 2), (4, 2)]
                for t, vr in [(1, 128), (3, 5), (16, 127), (20, 128), (33, 1), (64, 64)]
                if t <= 16 * mi]


@pytest.mark.parametrize("MI,KS,T,vrows", STREAM_CASES)
@pytest.mark.parametrize("packed", [False, True])
def test_stream_reads_inside_operands(MI, KS, T, vrows, packed):
    H = 256
    fa, fb = model_stream(MI, KS, packed, T, H, vrows)
    check_k_contiguous(fa, T, H, 0, H, f"stream hidden MI={MI} KS={KS}")
    if packed:  # a unit is 128 H contiguous elements, all of them read once
        a = fb.all()
        assert a.min() >= 0 and (a + 16).max() <= 128 * H * 2
        assert np.array_equal(np.unique(a), np.arange(0, 128 * H * 2, 16)) and a.size == 128 * H // 8
    else:
        check_k_contiguous(fb, vrows, H, 0, H, f"stream W MI={MI} KS={KS}")
