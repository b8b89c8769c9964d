"""Pins for the oracle's LayerNorm (CPU only).

The pages name LayerNorm as the first kernel of their LayerNorm -> Linear ->
GELU fusion example ("Lecture 6: GPU Kernels and Triton", section 6.1) but
print no formula; the oracle implements the standard definition (mean,
biased variance, eps inside the square root, per-column gamma and beta,
optional tanh-GELU after). It is pinned here against:
  * torch's own layer_norm in float64 (an independent implementation), with
    and without affine parameters, and with torch's tanh-approximate GELU;
  * invariants: normalised rows have mean 0 and variance var / (var + eps);
    shifting a row by a constant or scaling it (eps = 0) leaves the output;
  * closed forms: a constant row gives beta exactly; a two-column row [a, b]
    gives +-d / sqrt(d^2 + eps), d = (a - b) / 2;
  * fp32 / bf16 outputs are the double result rounded once.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

RNG = np.random.default_rng(2024)


def _torch_ln(x, g=None, b=None, eps=1e-5, gelu=False):
    t = torch.from_numpy(np.asarray(x, np.float64))
    y = F.layer_norm(t, (t.shape[-1],), None if g is None else torch.from_numpy(g),
                     None if b is None else torch.from_numpy(b), eps=eps)
    if gelu:
        y = F.gelu(y, approximate="tanh")
    return y.numpy()


@pytest.mark.parametrize("cols", [1, 2, 3, 17, 1000, 4096])
@pytest.mark.parametrize("affine", [False, True])
def test_matches_torch_layer_norm_in_double(cols, affine):
    x = RNG.standard_normal((9, cols)) * 3 + RNG.standard_normal((9, 1)) * 10
    g = RNG.standard_normal(cols) if affine else None
    b = RNG.standard_normal(cols) if affine else None
    got = oracle.layernorm_rows(x, g, b, eps=1e-5)
    assert np.allclose(got, _torch_ln(x, g, b), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("eps", [0.0, 1e-5, 1e-2, 1.0])
def test_eps_inside_the_square_root(eps):
    x = RNG.standard_normal((4, 50)) * 0.1
    got = oracle.layernorm_rows(x, eps=eps)
    assert np.allclose(got, _torch_ln(x, eps=eps), rtol=1e-12, atol=1e-12)


def test_gelu_epilogue_matches_torch():
    x = RNG.standard_normal((7, 333)) * 2
    g, b = RNG.standard_normal(333), RNG.standard_normal(333)
    got = oracle.layernorm_rows(x, g, b, gelu=True)
    assert np.allclose(got, _torch_ln(x, g, b, gelu=True), rtol=1e-12, atol=1e-12)


def test_normalised_rows_have_zero_mean_and_shrunk_unit_variance():
    x = RNG.standard_normal((20, 777)) * 5 + 30
    eps = 1e-3
    y = oracle.layernorm_rows(x, eps=eps)
    var = x.var(axis=1)
    assert np.abs(y.mean(axis=1)).max() < 1e-12
    assert np.allclose(y.var(axis=1), var / (var + eps), rtol=1e-12)


def test_shift_and_scale_invariance():
    x = RNG.standard_normal((6, 500))
    base = oracle.layernorm_rows(x, eps=0.0)
    assert np.allclose(oracle.layernorm_rows(x + 1234.5, eps=0.0), base, atol=1e-9)
    assert np.allclose(oracle.layernorm_rows(x * 37.0, eps=0.0), base, atol=1e-12)


def test_constant_row_gives_beta_exactly():
    b = RNG.standard_normal(1000)
    g = RNG.standard_normal(1000)
    x = np.full((3, 1000), 2.5)
    assert np.array_equal(oracle.layernorm_rows(x, g, b), np.broadcast_to(b, (3, 1000)))
    assert np.array_equal(oracle.layernorm_rows(x), np.zeros((3, 1000)))


def test_two_column_closed_form():
    a, b = RNG.standard_normal(50) * 4, RNG.standard_normal(50) * 4
    x = np.stack([a, b], axis=1)
    eps = 1e-5
    d = (a - b) / 2
    want = np.stack([d, -d], axis=1) / np.sqrt(d * d + eps)[:, None]
    assert np.allclose(oracle.layernorm_rows(x, eps=eps), want, rtol=1e-13, atol=1e-15)


def test_fp32_and_bf16_are_the_double_result_rounded_once():
    x32 = (RNG.standard_normal((8, 300)) * 3 + 80).astype(np.float32)
    g32 = (1 + 0.1 * RNG.standard_normal(300)).astype(np.float32)
    b32 = (0.1 * RNG.standard_normal(300)).astype(np.float32)
    d = oracle.layernorm_rows(x32.astype(np.float64), g32.astype(np.float64),
                              b32.astype(np.float64), gelu=True)
    assert np.array_equal(oracle.layernorm_rows(x32, g32, b32, gelu=True), d.astype(np.float32))
    xb, gb, bb = (oracle.f32_to_bf16(a) for a in (x32, g32, b32))
    db = oracle.layernorm_rows(oracle.bf16_to_f32(xb).astype(np.float64),
                               oracle.bf16_to_f32(gb).astype(np.float64),
                               oracle.bf16_to_f32(bb).astype(np.float64))
    assert np.array_equal(oracle.layernorm_rows(xb, gb, bb),
                          oracle.f32_to_bf16(db.astype(np.float32)))


def test_thread_count_does_not_change_bits():
    x = (RNG.standard_normal((101, 257)) * 2).astype(np.float32)
    assert np.array_equal(oracle.layernorm_rows(x, threads=1), oracle.layernorm_rows(x, threads=7))


def test_invalid_arguments():
    with pytest.raises(ValueError):
        oracle.layernorm_rows(np.zeros((2, 3)), eps=-1.0)
    with pytest.raises(ValueError):
        oracle.layernorm_rows(np.zeros((2, 3)), gamma=np.ones(4))
