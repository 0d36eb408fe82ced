"""Pins of the float64 LoRA-linear oracle (CPU).

The oracle (oracle/lora_linear.py) writes out y = x W^T + s (x A^T) B^T and
its gradients. Nothing here re-types those formulas: the forward is pinned by
closed forms and by the merged-weight form x (W + s B A)^T that the layer
stands for; the gradients by central finite differences of the scalar
L = sum(dy * y); the page's error measure by known cases.
"""

import numpy as np
import pytest
import torch

import workloads as wl
from oracle import lora_backward, lora_forward, rel_err

RNG = np.random.default_rng(1234)


def rnd(*shape):
    return RNG.standard_normal(shape)


def test_identity_base_and_zero_adapter_pass_x_through():
    x = rnd(5, 8)
    out = lora_forward(x, np.eye(8), np.zeros((3, 8)), rnd(8, 3), 2.0)
    assert np.array_equal(out["y"], x)
    assert np.array_equal(out["u"], np.zeros((5, 3)))


def test_rank_one_adapter_on_zero_base():
    x, a, b = rnd(4, 6), rnd(6), rnd(7)
    y = lora_forward(x, np.zeros((7, 6)), a[None, :], b[:, None], 0.5)["y"]
    want = 0.5 * np.outer(x @ a, b)  # y_t = s (x_t . a) b
    np.testing.assert_allclose(y, want, rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("scale", [1.0, 2.0, -0.75])
def test_merged_weight_form(scale):
    x, W, A, B = rnd(9, 12), rnd(10, 12), rnd(3, 12), rnd(10, 3)
    merged = W + scale * (B @ A)
    np.testing.assert_allclose(lora_forward(x, W, A, B, scale)["y"], x @ merged.T, rtol=1e-12,
                               atol=1e-12)


@pytest.mark.parametrize("scale", [1.0, 2.0])
def test_gradients_by_central_differences(scale):
    T, K, N, r = 3, 5, 4, 2
    x, W, A, B, dy = rnd(T, K), rnd(N, K), rnd(r, K), rnd(N, r), rnd(T, N)
    g = lora_backward(x, W, A, B, dy, scale)

    def loss(x_, A_, B_):
        return float(np.sum(dy * lora_forward(x_, W, A_, B_, scale)["y"]))

    h = 1e-6
    for name, arr in (("dx", x), ("dA", A), ("dB", B)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            p, m = arr.copy(), arr.copy()
            p[idx] += h
            m[idx] -= h
            args = {"dx": (p, A, B), "dA": (x, p, B), "dB": (x, A, p)}[name]
            argm = {"dx": (m, A, B), "dA": (x, m, B), "dB": (x, A, m)}[name]
            num[idx] = (loss(*args) - loss(*argm)) / (2 * h)
        np.testing.assert_allclose(g[name], num, rtol=1e-7, atol=1e-8, err_msg=name)


def test_no_gradient_for_the_frozen_base():
    x, W, A, B, dy = rnd(2, 4), rnd(3, 4), rnd(1, 4), rnd(3, 1), rnd(2, 3)
    assert set(lora_backward(x, W, A, B, dy)) == {"dx", "dA", "dB"}


def test_rows_are_independent():
    c = wl.lora_case(64, 128, 20, 7)
    full = lora_forward(c.x, c.W, c.A, c.B, 2.0)["y"]
    part = lora_forward(c.x[5:9], c.W, c.A, c.B, 2.0)["y"]
    np.testing.assert_allclose(part, full[5:9], rtol=1e-14, atol=1e-14)
    gfull = lora_backward(c.x, c.W, c.A, c.B, c.dy, 2.0)["dx"]
    gpart = lora_backward(c.x[5:9], c.W, c.A, c.B, c.dy[5:9], 2.0)["dx"]
    np.testing.assert_allclose(gpart, gfull[5:9], rtol=1e-14, atol=1e-14)


def test_rel_err_known_cases():
    a = rnd(7, 3)
    assert rel_err(a, a) == 0.0
    assert abs(rel_err(1.001 * a, a) - 1e-3) < 1e-12
    assert abs(rel_err(np.zeros_like(a), a) - 1.0) < 1e-15
    # bf16 rounding of an N(0,1) tensor: the scale of the page's forward and
    # grad_x errors (1.66e-3), which a bf16 output cannot beat
    t = torch.randn(512, 512, generator=torch.Generator().manual_seed(3))
    e = rel_err(t.to(torch.bfloat16), t.double().numpy())
    assert 1.0e-3 < e < 2.5e-3, e


def test_bf16_inputs_decode_exactly():
    c = wl.lora_case(64, 64, 3, 8)
    y = lora_forward(c.x, c.W, c.A, c.B)["y"]
    ref = lora_forward(c.x.double().numpy(), c.W.double().numpy(), c.A.double().numpy(),
                       c.B.double().numpy())["y"]
    assert np.array_equal(y, ref)
