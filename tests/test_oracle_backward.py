"""Pins for the oracle's backward functions (CPU only).

The pages print no backward formulas; the oracle derives them from the
forward definitions (tanh-GELU of the "CS336 lecture 6" notes, section 4.2;
row softmax of section 5.2). Pinned here against:
  * torch autograd in float64 (an independent implementation);
  * central finite differences of the oracle's own forward functions (which
    are pinned in their own tests), so the derivative is tied to the
    forward definition;
  * special values and identities: GELU'(0) = 1/2, limits 1 and 0 at +-inf,
    the sign change at GELU's minimum; softmax: dx sums to 0 over a row,
    a constant dy or a one-hot y gives dx = 0, and <dx, v> = <dy, J v>.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

RNG = np.random.default_rng(77)


def torch_gelu_grad(x):
    t = torch.from_numpy(np.asarray(x, np.float64)).requires_grad_(True)
    F.gelu(t, approximate="tanh").sum().backward()
    return t.grad.numpy()


def test_gelu_grad_matches_torch_autograd():
    x = np.linspace(-8.0, 8.0, 40001)
    g = oracle.gelu_tanh_grad_f64(x)
    assert np.abs(g - torch_gelu_grad(x)).max() < 1e-13
    # where torch's 1 + tanh does not cancel, also relatively
    m = x > -3
    t = torch_gelu_grad(x[m])
    assert np.max(np.abs(g[m] - t) / np.maximum(np.abs(t), 1e-300)) < 1e-11


def test_gelu_grad_is_the_derivative_of_the_forward():
    x = RNG.uniform(-9.0, 9.0, 5000)
    h = 1e-5
    fd = (oracle.gelu_tanh_f64(x + h) - oracle.gelu_tanh_f64(x - h)) / (2 * h)
    assert np.abs(fd - oracle.gelu_tanh_grad_f64(x)).max() < 1e-8


def test_gelu_grad_special_values():
    g = oracle.gelu_tanh_grad_f64(np.array([0.0, np.inf, -np.inf, np.nan, 12.0, 40.0, -40.0]))
    assert g[0] == 0.5
    assert g[1] == 1.0 and g[2] == 0.0 and np.isnan(g[3])
    assert abs(g[4] - 1.0) < 1e-15 and g[5] == 1.0
    assert abs(g[6]) < 1e-300
    # GELU has a single minimum near x = -0.75: GELU' changes sign there
    assert oracle.gelu_tanh_grad_f64(np.array([-0.80]))[0] < 0 < oracle.gelu_tanh_grad_f64(
        np.array([-0.70]))[0]


def test_gelu_bwd_is_the_double_product_rounded_once():
    x = (RNG.standard_normal(20000) * 3).astype(np.float32)
    dy = RNG.standard_normal(20000).astype(np.float32)
    want = (dy.astype(np.float64) * oracle.gelu_tanh_grad_f64(x)).astype(np.float32)
    assert np.array_equal(oracle.gelu_tanh_backward(x, dy), want)
    xb, dyb = oracle.f32_to_bf16(x), oracle.f32_to_bf16(dy)
    wantb = oracle.f32_to_bf16((oracle.bf16_to_f32(dyb).astype(np.float64)
                                * oracle.gelu_tanh_grad_f64(oracle.bf16_to_f32(xb)))
                               .astype(np.float32))
    assert np.array_equal(oracle.gelu_tanh_backward(xb, dyb), wantb)


@pytest.mark.parametrize("cols", [1, 2, 7, 1000])
def test_softmax_bwd_matches_torch_autograd(cols):
    x = RNG.standard_normal((6, cols)) * 3
    dy = RNG.standard_normal((6, cols))
    tx = torch.from_numpy(x).requires_grad_(True)
    ty = torch.softmax(tx, dim=1)
    ty.backward(torch.from_numpy(dy))
    dx = oracle.softmax_rows_backward(ty.detach().numpy(), dy)
    assert np.abs(dx - tx.grad.numpy()).max() < 1e-15


def test_softmax_bwd_identities():
    x = RNG.standard_normal((8, 300)) * 2
    y = oracle.softmax_rows(x)
    dy = RNG.standard_normal((8, 300))
    dx = oracle.softmax_rows_backward(y, dy)
    assert np.abs(dx.sum(axis=1)).max() < 1e-15                     # rows of J^T sum to 0
    const = oracle.softmax_rows_backward(y, np.full_like(y, 3.25))
    assert np.abs(const).max() < 1e-15                               # J^T 1 = 0
    onehot = np.zeros_like(y)
    onehot[np.arange(8), RNG.integers(0, 300, 8)] = 1.0
    assert np.array_equal(oracle.softmax_rows_backward(onehot, dy), np.zeros_like(y))
    # <dx, v> = <dy, J v>, J v by central differences of the forward softmax
    v = RNG.standard_normal((8, 300))
    h = 1e-6
    jv = (oracle.softmax_rows(x + h * v) - oracle.softmax_rows(x - h * v)) / (2 * h)
    assert np.allclose((dx * v).sum(axis=1), (dy * jv).sum(axis=1), rtol=1e-7, atol=1e-10)


def test_softmax_bwd_fp32_and_bf16_round_the_double_result():
    y32 = oracle.softmax_rows((RNG.standard_normal((5, 257)) * 2).astype(np.float32))
    dy32 = RNG.standard_normal((5, 257)).astype(np.float32)
    d = oracle.softmax_rows_backward(y32.astype(np.float64), dy32.astype(np.float64))
    assert np.array_equal(oracle.softmax_rows_backward(y32, dy32), d.astype(np.float32))
    yb, dyb = oracle.f32_to_bf16(y32), oracle.f32_to_bf16(dy32)
    db = oracle.softmax_rows_backward(oracle.bf16_to_f32(yb).astype(np.float64),
                                      oracle.bf16_to_f32(dyb).astype(np.float64))
    assert np.array_equal(oracle.softmax_rows_backward(yb, dyb),
                          oracle.f32_to_bf16(db.astype(np.float32)))
