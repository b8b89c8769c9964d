"""Pins for the oracle's tanh-GELU (CPU only).

The definition is the tanh form of the "CS336 lecture 6" notes (kyc001),
section 4.2. Each pin is chosen so that a plausible slip in the oracle --
a dropped cubic term, a wrong power or sign, a lost factor 0.5, a bad
constant, a wrong rounding -- fails at least one of them:

* torch's own ``F.gelu(approximate="tanh")`` in float64 (an independent
  implementation of the same definition);
* the exact erf-GELU x * Phi(x) from ``math.erf``, which the tanh form fits
  to within 4.73e-4 (a dropped cubic term is off by 3.4e-2);
* the odd identity GELU(x) - GELU(-x) = x, from tanh being odd;
* GELU(+-0) = +-0, GELU(x) = x in fp32 for large x, GELU -> -0 for x -> -inf;
* the literal 0.5x(1+tanh u) and the cancellation-free x/(1+exp(-2u)) agree
  where the literal form is accurate in double.
"""
import math

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _torch_gelu64(x):
    return torch.nn.functional.gelu(torch.from_numpy(np.asarray(x, np.float64)),
                                    approximate="tanh").numpy()


def _ulp_diff_f32(a, b):
    """Distance in fp32 ulps through the monotone integer order of the bit patterns."""
    ia = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    ib = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    ia = np.where(ia < 0, -(ia & 0x7FFFFFFF), ia)
    ib = np.where(ib < 0, -(ib & 0x7FFFFFFF), ib)
    return np.abs(ia - ib)


def test_matches_torch_tanh_gelu_in_double():
    # torch evaluates the literal form; in double it is accurate to ~1e-13
    # relative down to x = -3 and to ~1e-9 down to x = -4.5.
    x = np.linspace(-3.0, 12.0, 150_001)
    r = oracle.gelu_tanh_f64(x)
    t = _torch_gelu64(x)
    nz = x != 0
    assert np.max(np.abs(r[nz] - t[nz]) / np.abs(t[nz])) < 1e-12
    x2 = np.linspace(-4.5, -3.0, 10_001)
    r2, t2 = oracle.gelu_tanh_f64(x2), _torch_gelu64(x2)
    assert np.max(np.abs(r2 - t2) / np.abs(t2)) < 1e-9


def test_close_to_erf_gelu():
    x = np.linspace(-10.0, 10.0, 400_001)
    exact = np.array([0.5 * v * (1.0 + math.erf(v / math.sqrt(2.0))) for v in x[::40]])
    d = np.abs(oracle.gelu_tanh_f64(x[::40]) - exact)
    assert d.max() < 5e-4           # the tanh fit's own error is 4.73e-4
    assert d.max() > 4e-4           # and it is an approximation, not erf itself


def test_odd_identity():
    x = np.concatenate([np.linspace(-12, 12, 240_001), [1e-30, 1e-8, 3.5, 7.25]])
    g = oracle.gelu_tanh_f64(x)
    gm = oracle.gelu_tanh_f64(-x)
    # GELU(x) - GELU(-x) = x, up to a few double roundings of the terms
    err = np.abs(g - gm - x)
    assert np.all(err <= 4e-16 * (np.abs(g) + np.abs(gm)) + 1e-300)


def test_signed_zero_and_specials():
    x = np.array([0.0, -0.0, np.inf, -np.inf, np.nan], np.float32)
    y = oracle.gelu_tanh(x)
    assert y[0] == 0 and not np.signbit(y[0])
    assert y[1] == 0 and np.signbit(y[1])
    assert y[2] == np.inf
    assert y[3] == 0 and np.signbit(y[3])      # reading: the limit, -0
    assert np.isnan(y[4])


def test_large_positive_is_identity_in_fp32():
    # 1 - (1 + tanh u)/2 < 3e-11 for x >= 6, far below half an fp32 ulp.
    x = np.linspace(6.0, 3.0e38, 100_001, dtype=np.float32)
    x = np.concatenate([x, np.float32([6.0, 7.5, 100.0, 1e20, np.finfo(np.float32).max])])
    assert np.array_equal(oracle.gelu_tanh(x).view(np.uint32), x.view(np.uint32))


def test_large_negative_goes_to_minus_zero():
    x = -np.geomspace(30.0, 3.0e38, 10_001).astype(np.float32)
    y = oracle.gelu_tanh(x)
    assert np.all(y == 0) and np.all(np.signbit(y))
    # and on (-12, 0) it is strictly negative until it underflows
    x2 = np.linspace(-9.9, -1e-6, 10_001).astype(np.float32)
    assert np.all(oracle.gelu_tanh(x2) < 0)


def test_tiny_outputs_keep_relative_accuracy():
    # The literal double form returns exactly 0 below about -7.3; the oracle
    # must not: GELU(-9) ~ -1.34e-28, still a normal fp32 number.
    y = oracle.gelu_tanh_f64(np.array([-9.0]))[0]
    assert -1.4e-28 < y < -1.3e-28
    lit = oracle.gelu_tanh_literal_f64(np.array([-9.0]))[0]
    assert lit == 0.0 or abs(lit - y) > 1e-3 * abs(y)


def test_literal_and_identity_forms_agree():
    x = np.linspace(-3.0, 10.0, 130_001)
    a, b = oracle.gelu_tanh_f64(x), oracle.gelu_tanh_literal_f64(x)
    nz = x != 0
    assert np.max(np.abs(a[nz] - b[nz]) / np.abs(a[nz])) < 1e-12


def test_fp32_result_is_the_rounded_double():
    # Independent of the oracle's rounding code path: numpy's own float64 ->
    # float32 rounding of torch's double GELU. Both doubles are within 1e-12
    # relative, so the fp32 results are within one ulp (equal in practice).
    rng = np.random.default_rng(7)
    x = rng.uniform(-3, 8, 200_000).astype(np.float32)
    ref = _torch_gelu64(x.astype(np.float64)).astype(np.float32)
    got = oracle.gelu_tanh(x)
    d = _ulp_diff_f32(got, ref)
    assert d.max() <= 1
    assert (d == 0).mean() > 0.9999


def test_bf16_is_fp32_result_rounded_to_bf16():
    # torch's float32 -> bfloat16 (nearest even) applied to the fp32 oracle.
    rng = np.random.default_rng(8)
    xf = rng.standard_normal(100_000).astype(np.float32)
    xb = torch.from_numpy(xf).to(torch.bfloat16)
    xb_bits = xb.view(torch.int16).numpy().view(np.uint16)
    y = oracle.gelu_tanh(xb_bits)
    yf32 = oracle.gelu_tanh(xb.float().numpy())
    ref = torch.from_numpy(yf32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(y, ref)


def test_thread_count_does_not_change_bits():
    rng = np.random.default_rng(9)
    x = rng.standard_normal(300_001).astype(np.float32)
    a = oracle.gelu_tanh(x, threads=1)
    b = oracle.gelu_tanh(x, threads=7)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
