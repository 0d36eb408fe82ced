"""Pins of the float64 oracle against things other than itself (CPU only).

Each test fixes part of the oracle by a closed form, an independent
high-precision computation (exact rationals + 50-digit decimals), finite
differences or an invariant, so that a dropped term, a wrong sign or index or
a transposed operand anywhere in ``oracle/`` fails at least one of them.
"""

import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import expit, log_expit

from oracle import (backward_f64, decode_bf16, finalize_partials, forward, forward_f64,
                    merge_partials, slice_partials_f64)
from oracle import brute

HERE = os.path.dirname(os.path.abspath(__file__))


def rng(seed):
    return np.random.default_rng(seed)


def bf16_round_np(x):
    return decode_bf16(torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16))


# ---------------------------------------------------------------- decoding

def test_decode_bf16_bit_patterns():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x7F80, 0x0001, 0x3F81, 0x4049], np.uint16)
    got = decode_bf16(bits)
    want = [1.0, -2.0, 0.0, -0.0, math.inf, 2.0 ** -133, 1.0 + 2.0 ** -7, 3.140625]
    assert got.tolist() == want
    assert math.copysign(1.0, got[3]) == -1.0


def test_decode_bf16_matches_torch_roundtrip():
    x = torch.randn(1000, generator=torch.Generator().manual_seed(0)) * 100
    b = x.to(torch.bfloat16)
    assert np.array_equal(decode_bf16(b), b.double().numpy())


# ------------------------------------------------------------ closed forms

@pytest.mark.parametrize("V", [2, 7, 1024])
def test_uniform_logits_zero_weight(V):
    h = rng(1).standard_normal((5, 16))
    W = np.zeros((V, 16))
    y = rng(2).integers(0, V, 5)
    o = forward_f64(h, W, y)
    np.testing.assert_allclose(o["logp"], -math.log(V), rtol=1e-15, atol=0)
    np.testing.assert_allclose(o["entropy"], math.log(V), rtol=1e-14, atol=0)


def test_uniform_logits_identical_rows():
    V, H = 333, 24
    w = rng(3).standard_normal(H)
    W = np.tile(w, (V, 1))
    h = rng(4).standard_normal((6, H))
    y = rng(5).integers(0, V, 6)
    o = forward_f64(h, W, y)
    np.testing.assert_allclose(o["logp"], -math.log(V), rtol=1e-14)
    np.testing.assert_allclose(o["entropy"], math.log(V), rtol=1e-13)


@pytest.mark.parametrize("c", [64.0, 4.0, 0.5])
def test_one_hot_dominant(c):
    # hidden row = a e0, W[y] = b e0 (a b = c), others 0: z_y = c, rest 0.
    # With q = (V-1) e^{-c}:  logp = -log1p(q),  H = log1p(q) + c q / (1+q).
    V, H, T = 1024, 8, 3
    a = math.sqrt(c)
    h = np.zeros((T, H)); h[:, 0] = a
    y = np.array([0, 511, 1023])
    o_logp, o_ent = [], []
    for t in range(T):
        W = np.zeros((V, H)); W[y[t], 0] = a
        o = forward_f64(h[t:t + 1], W, y[t:t + 1])
        o_logp.append(o["logp"][0]); o_ent.append(o["entropy"][0])
    q = (V - 1) * math.exp(-c)
    np.testing.assert_allclose(o_logp, -math.log1p(q), rtol=1e-12)
    np.testing.assert_allclose(o_ent, math.log1p(q) + c * q / (1 + q), rtol=1e-12)
    if c == 64.0:
        assert abs(o_logp[0]) < 1e-20 and 0 < o_ent[0] < 1e-20


def test_two_class_reduces_to_logistic():
    # V = 2: logp = log sigmoid(z_y - z_other); H = binary entropy of sigmoid.
    r = rng(6)
    h = r.standard_normal((50, 4)) * 3
    W = r.standard_normal((2, 4))
    y = r.integers(0, 2, 50)
    o = forward_f64(h, W, y)
    z = h @ W.T
    s = z[np.arange(50), y] - z[np.arange(50), 1 - y]
    np.testing.assert_allclose(o["logp"], log_expit(s), rtol=1e-13, atol=1e-300)
    hb = -(expit(s) * log_expit(s) + expit(-s) * log_expit(-s))
    np.testing.assert_allclose(o["entropy"], hb, rtol=1e-12)


# ---------------------------------------------------------- brute force

@pytest.mark.parametrize("V,scale,seed", [(3, 1, 0), (17, 1, 1), (64, 1, 2), (64, 8, 3), (64, 40, 4)])
def test_forward_matches_exact_brute_force(V, scale, seed):
    r = rng(seed)
    T, H = 4, 8
    h = bf16_round_np(r.standard_normal((T, H)))
    W = bf16_round_np(r.standard_normal((V, H)) * 0.3 * scale)
    y = r.integers(0, V, T)
    o = forward_f64(h, W, y)
    bl, be = brute.logp_entropy(h, W, y)
    for t in range(T):
        assert abs(o["logp"][t] - float(bl[t])) <= 1e-13 * max(1.0, abs(float(bl[t])))
        assert abs(o["entropy"][t] - float(be[t])) <= 1e-13 * abs(float(be[t])) + 1e-300


def test_golden_fixture():
    """Stored 30-digit brute-force values (tests/golden/make_golden.py)."""
    with open(os.path.join(HERE, "golden", "tiny_bruteforce.json")) as f:
        g = json.load(f)
    h = decode_bf16(np.array(g["hidden_bits"], dtype=np.uint16).reshape(g["T"], g["H"]))
    W = decode_bf16(np.array(g["weight_bits"], dtype=np.uint16).reshape(g["V"], g["H"]))
    o = forward_f64(h, W, np.array(g["targets"]))
    want_l = np.array([float(s) for s in g["logp"]])
    want_e = np.array([float(s) for s in g["entropy"]])
    np.testing.assert_allclose(o["logp"], want_l, rtol=1e-13)
    np.testing.assert_allclose(o["entropy"], want_e, rtol=1e-13)


# ---------------------------------------------- gradients: finite differences

def _loss(h, W, y, gl, ge):
    o = forward_f64(h, W, y)
    return float(gl @ o["logp"] + ge @ o["entropy"])


@pytest.mark.parametrize("which", ["logp", "entropy", "both"])
def test_gradients_match_finite_differences(which):
    r = rng(11)
    T, H, V = 3, 5, 7
    h = r.standard_normal((T, H))
    W = r.standard_normal((V, H)) * 0.7
    y = np.array([0, 3, 6])
    gl = r.standard_normal(T) if which in ("logp", "both") else np.zeros(T)
    ge = r.standard_normal(T) if which in ("entropy", "both") else np.zeros(T)
    g = backward_f64(h, W, y, gl, ge)
    eps = 1e-6
    fdH = np.zeros_like(h)
    for i in np.ndindex(h.shape):
        hp, hm = h.copy(), h.copy(); hp[i] += eps; hm[i] -= eps
        fdH[i] = (_loss(hp, W, y, gl, ge) - _loss(hm, W, y, gl, ge)) / (2 * eps)
    fdW = np.zeros_like(W)
    for i in np.ndindex(W.shape):
        Wp, Wm = W.copy(), W.copy(); Wp[i] += eps; Wm[i] -= eps
        fdW[i] = (_loss(h, Wp, y, gl, ge) - _loss(h, Wm, y, gl, ge)) / (2 * eps)
    assert np.linalg.norm(g["dH"] - fdH) <= 1e-6 * np.linalg.norm(fdH)
    assert np.linalg.norm(g["dW"] - fdW) <= 1e-6 * np.linalg.norm(fdW)


def test_gradient_closed_form_zero_hidden():
    # h = 0: uniform softmax, so dH_t = dlogp_t (w_{y_t} - mean_v w_v), dW = 0
    # (the entropy gradient vanishes at the uniform distribution).
    r = rng(12)
    T, H, V = 4, 6, 9
    W = r.standard_normal((V, H))
    y = np.array([1, 8, 0, 1])
    gl, ge = r.standard_normal(T), r.standard_normal(T)
    g = backward_f64(np.zeros((T, H)), W, y, gl, ge)
    want = gl[:, None] * (W[y] - W.mean(axis=0))
    np.testing.assert_allclose(g["dH"], want, rtol=1e-13, atol=1e-14)
    assert np.abs(g["dW"]).max() == 0.0


def test_gradient_closed_form_identical_rows():
    # identical W rows: uniform softmax, dH = 0 and
    # dW[v] = sum_t dlogp_t ([v == y_t] - 1/V) h_t.
    r = rng(13)
    T, H, V = 5, 4, 6
    W = np.tile(r.standard_normal(H), (V, 1))
    h = r.standard_normal((T, H))
    y = np.array([0, 0, 2, 5, 3])
    gl, ge = r.standard_normal(T), r.standard_normal(T)
    g = backward_f64(h, W, y, gl, ge)
    assert np.abs(g["dH"]).max() < 1e-14
    onehot = np.eye(V)[y]
    want = (gl[:, None] * (onehot - 1.0 / V)).T @ h
    np.testing.assert_allclose(g["dW"], want, rtol=1e-12, atol=1e-14)


# --------------------------------------------------------------- invariants

def _rand_case(seed, T=8, H=16, V=50, scale=1.0):
    r = rng(seed)
    return (r.standard_normal((T, H)), r.standard_normal((V, H)) * scale,
            r.integers(0, V, T), r.standard_normal(T), r.standard_normal(T))


def test_shift_invariance():
    h, W, y, _, _ = _rand_case(20)
    shift = rng(21).standard_normal(W.shape[1])
    a = forward_f64(h, W, y)
    b = forward_f64(h, W + shift, y)
    np.testing.assert_allclose(a["logp"], b["logp"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(a["entropy"], b["entropy"], rtol=1e-12, atol=1e-12)


def test_vocab_permutation_equivariance():
    h, W, y, gl, ge = _rand_case(22)
    perm = rng(23).permutation(W.shape[0])
    inv = np.argsort(perm)
    a = forward_f64(h, W, y)
    b = forward_f64(h, W[perm], inv[y])
    np.testing.assert_allclose(a["logp"], b["logp"], rtol=1e-13)
    np.testing.assert_allclose(a["entropy"], b["entropy"], rtol=1e-13)
    ga = backward_f64(h, W, y, gl, ge)
    gb = backward_f64(h, W[perm], inv[y], gl, ge)
    np.testing.assert_allclose(ga["dH"], gb["dH"], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(ga["dW"][perm], gb["dW"], rtol=1e-12, atol=1e-13)


def test_bounds_and_column_sum():
    h, W, y, gl, ge = _rand_case(24, T=20, V=80, scale=3.0)
    o = forward_f64(h, W, y)
    assert (o["logp"] <= 0).all()
    assert (o["entropy"] >= 0).all() and (o["entropy"] <= math.log(80) + 1e-12).all()
    g = backward_f64(h, W, y, gl, ge)
    # sum_v G[t,v] = 0 for every row, so the columns of dW sum to zero
    assert np.abs(g["dW"].sum(axis=0)).max() <= 1e-12 * np.abs(g["dW"]).max()


def test_logp_exp_sums_to_one():
    # exp(logp) over every possible target sums to 1 for each row
    h, W, _, _, _ = _rand_case(25, T=3, V=40, scale=2.0)
    tot = np.zeros(3)
    for v in range(40):
        tot += np.exp(forward_f64(h, W, np.full(3, v))["logp"])
    np.testing.assert_allclose(tot, 1.0, rtol=1e-13)


# ------------------------------------------------------ slices and merging

@pytest.mark.parametrize("seed", [30, 31, 32])
def test_slice_combine_equals_full(seed):
    r = rng(seed)
    T, H, V = 12, 10, 97
    h = r.standard_normal((T, H))
    W = r.standard_normal((V, H)) * (1.0 + 4 * (seed - 30))
    y = r.integers(0, V, T)
    full = forward_f64(h, W, y)
    cuts = np.sort(r.choice(np.arange(1, V), size=5, replace=False))
    bounds = [0, *cuts.tolist(), V]
    parts = [slice_partials_f64(h, W[a:b], y, a) for a, b in zip(bounds[:-1], bounds[1:])]
    order = r.permutation(len(parts))
    acc = parts[order[0]]
    for i in order[1:]:
        acc = merge_partials(acc, parts[i])
    fin = finalize_partials(acc)
    np.testing.assert_allclose(fin["logp"], full["logp"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(fin["entropy"], full["entropy"], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(fin["lse"], full["lse"], rtol=1e-13)


def test_slice_partial_single_column_and_ties():
    # one-column slice: m = z, R = 0, B = 0; a slice of equal logits: R = n - 1, B = 0
    h = np.ones((2, 3))
    W = np.array([[1.0, 2.0, 3.0], [0.5, 0.5, 0.5], [0.5, 0.5, 0.5], [0.5, 0.5, 0.5]])
    m, R, B, zy = slice_partials_f64(h, W[:1], np.array([0, 2]), 0)
    assert m.tolist() == [6.0, 6.0] and R.tolist() == [0.0, 0.0] and B.tolist() == [0.0, 0.0]
    assert zy[0] == 6.0 and np.isneginf(zy[1])
    m, R, B, zy = slice_partials_f64(h, W[1:], np.array([0, 2]), 1)
    assert R.tolist() == [2.0, 2.0] and B.tolist() == [0.0, 0.0]
    assert np.isneginf(zy[0]) and zy[1] == 1.5


def test_backward_vocab_range_partition():
    h, W, y, gl, ge = _rand_case(33, T=6, V=45)
    full = backward_f64(h, W, y, gl, ge)
    acc = np.zeros_like(full["dH"])
    for a, b in [(0, 11), (11, 30), (30, 45)]:
        part = backward_f64(h, W, y, gl, ge, vocab_range=(a, b))
        acc += part["dH"]
        np.testing.assert_allclose(part["dW"], full["dW"][a:b], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(acc, full["dH"], rtol=1e-12, atol=1e-14)


def test_bf16_entry_points_decode_inputs():
    r = rng(40)
    hb = torch.from_numpy(r.standard_normal((5, 8)).astype(np.float32)).to(torch.bfloat16)
    Wb = torch.from_numpy(r.standard_normal((11, 8)).astype(np.float32)).to(torch.bfloat16)
    y = torch.tensor([0, 1, 2, 10, 5], dtype=torch.int32)
    a = forward(hb, Wb, y)
    b = forward_f64(hb.double().numpy(), Wb.double().numpy(), y.numpy())
    assert np.array_equal(a["logp"], b["logp"]) and np.array_equal(a["entropy"], b["entropy"])


# ------------------------------------ sampled rows of the backward (used by
# every full-size GPU gradient comparison) and the absolute-term sums

@pytest.mark.parametrize("vocab_range", [None, (7, 31)])
@pytest.mark.parametrize("with_dent", [False, True])
def test_backward_sampled_rows_equal_full_rows(vocab_range, with_dent):
    # rows spread over several row blocks, out of order; vocabulary rows out
    # of order, with repeats of target rows
    h, W, y, gl, ge = _rand_case(41, T=23, H=12, V=45, scale=1.5)
    ge = ge if with_dent else None
    full = backward_f64(h, W, y, gl, ge, vocab_range=vocab_range, with_abs=True, row_block=4)
    a, b = vocab_range or (0, 45)
    rows = np.array([17, 0, 5, 22, 8, 9])
    vrows = np.array([b - 1, a, a + 3, a + 9, a + 4]) if vocab_range else np.array([44, 0, int(y[3]), 9, 30])
    part = backward_f64(h, W, y, gl, ge, dh_rows=rows, dw_rows=vrows, vocab_range=vocab_range,
                        with_abs=True, row_block=4)
    assert np.array_equal(part["dh_rows"], rows) and np.array_equal(part["dw_rows"], vrows)
    np.testing.assert_allclose(part["dH"], full["dH"][rows], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(part["dW"], full["dW"][vrows - a], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(part["dH_abs"], full["dH_abs"][rows], rtol=1e-12, atol=0)
    np.testing.assert_allclose(part["dW_abs"], full["dW_abs"][vrows - a], rtol=1e-12, atol=0)
    # the row-block size does not change the rows
    one = backward_f64(h, W, y, gl, ge, dh_rows=rows, dw_rows=vrows, vocab_range=vocab_range,
                       row_block=256)
    np.testing.assert_allclose(one["dH"], part["dH"], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(one["dW"], part["dW"], rtol=1e-12, atol=1e-15)


def test_backward_sampled_rows_reject_rows_outside_the_range():
    h, W, y, gl, _ = _rand_case(42, T=4, V=20)
    with pytest.raises(ValueError):
        backward_f64(h, W, y, gl, dw_rows=np.array([3]), vocab_range=(5, 10))


def test_abs_terms_closed_form_uniform_softmax():
    # identical W rows give p = 1/V and log p + entropy = 0, so
    # G[t, v] = dlogp_t ([v == y_t] - 1/V):
    #   dH_abs[t, k] = |dlogp_t| sum_v |[v == y_t] - 1/V| |W[v, k]|
    #   dW_abs[v, k] = sum_t |dlogp_t| |[v == y_t] - 1/V| |h[t, k]|
    r = rng(43)
    T, H, V = 5, 4, 6
    W = np.tile(r.standard_normal(H), (V, 1))
    h = r.standard_normal((T, H))
    y = np.array([0, 0, 2, 5, 3])
    gl, ge = r.standard_normal(T), r.standard_normal(T)
    g = backward_f64(h, W, y, gl, ge, with_abs=True)
    coef = np.abs(gl)[:, None] * np.abs(np.eye(V)[y] - 1.0 / V)  # [T, V]
    np.testing.assert_allclose(g["dH_abs"], coef @ np.abs(W), rtol=1e-12)
    np.testing.assert_allclose(g["dW_abs"], coef.T @ np.abs(h), rtol=1e-12)


def test_abs_terms_bound_the_gradients():
    h, W, y, gl, ge = _rand_case(44, T=9, V=60, scale=2.0)
    g = backward_f64(h, W, y, gl, ge, with_abs=True)
    assert (np.abs(g["dH"]) <= g["dH_abs"] * (1 + 1e-12)).all()
    assert (np.abs(g["dW"]) <= g["dW_abs"] * (1 + 1e-12)).all()
    # mixed signs cancel: the bound is strict somewhere
    assert (np.abs(g["dH"]) < 0.999 * g["dH_abs"]).any()
