"""Pins for the oracle's row softmax (CPU only).

The definition: per row, the max, then exp(x - max) and its sum, then the
quotient ("CS336 lecture 6" notes (kyc001), section 5.2; "Lecture 6: GPU
Kernels and Triton", section 7.2). Pins independent of the oracle's code:

* torch.softmax in float64 (an independent implementation);
* scipy's logistic function for two-column rows;
* rows sum to 1; cols = 1 gives exactly 1; a constant row of 2^k columns
  gives exactly 2^-k;
* shift invariance with a shift so large (+800) that exp would overflow
  without the max subtraction; on exactly representable inputs the fp32
  results are bitwise identical;
* brute force on tiny shapes; strided rows leave padding untouched.
"""
import numpy as np
import pytest
import torch
from scipy.special import expit

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _torch_softmax64(x):
    return torch.softmax(torch.from_numpy(np.asarray(x, np.float64)), dim=-1).numpy()


def test_matches_torch_softmax_double():
    rng = np.random.default_rng(1)
    for rows, cols, scale in [(7, 1000, 3.0), (3, 4096, 8.0), (2, 131072, 2.0), (5, 33, 30.0)]:
        x = rng.standard_normal((rows, cols)) * scale
        r = oracle.softmax_rows(x)
        t = _torch_softmax64(x)
        assert np.max(np.abs(r - t)) < 1e-13    # summation order differs
        assert np.max(np.abs(r - t) / t) < 1e-12


def test_brute_force_tiny_shapes():
    rng = np.random.default_rng(2)
    for rows in (1, 3, 17):
        for cols in range(1, 41):
            x = rng.standard_normal((rows, cols)) * 4.0
            assert np.allclose(oracle.softmax_rows(x), _torch_softmax64(x), rtol=1e-12, atol=0)
            xf = x.astype(np.float32)
            ref = _torch_softmax64(xf.astype(np.float64)).astype(np.float32)
            got = oracle.softmax_rows(xf)
            assert np.max(np.abs(got - ref)) <= 6e-8


def test_rows_sum_to_one():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((64, 1000)) * 3).astype(np.float32)
    x[::16] += 80
    y = oracle.softmax_rows(x).astype(np.float64)
    assert np.max(np.abs(y.sum(axis=1) - 1.0)) < 1e-5
    y64 = oracle.softmax_rows(x.astype(np.float64))
    assert np.max(np.abs(y64.sum(axis=1) - 1.0)) < 1e-13


def test_two_columns_is_logistic():
    rng = np.random.default_rng(4)
    a, b = rng.standard_normal(1000) * 5, rng.standard_normal(1000) * 5
    y = oracle.softmax_rows(np.stack([a, b], axis=1))
    assert np.allclose(y[:, 0], expit(a - b), rtol=1e-13, atol=0)
    assert np.allclose(y[:, 1], expit(b - a), rtol=1e-13, atol=0)


def test_single_column_and_constant_rows():
    x = np.float32([[-3.0], [0.0], [1e30], [-1e30]])
    assert np.all(oracle.softmax_rows(x) == 1.0)
    for k in range(0, 14):
        cols = 1 << k
        x = np.full((3, cols), 2.5, np.float32)
        assert np.all(oracle.softmax_rows(x) == np.float32(1.0 / cols))


def test_shift_invariance_is_exact_and_needs_max_subtraction():
    rng = np.random.default_rng(5)
    # values on a 2^-10 grid with |x| < 2^10: x + 800 is exact in fp32
    x = (np.round(rng.standard_normal((32, 1000)) * 3 * 1024) / 1024).astype(np.float32)
    xs = x + np.float32(800.0)
    assert np.array_equal((xs - np.float32(800.0)), x)          # the shift is exact
    a, b = oracle.softmax_rows(x), oracle.softmax_rows(xs)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert np.all(np.isfinite(b))                               # exp(800) would overflow


def test_nonfinite_rows_follow_the_formula():
    x = np.float32([[1.0, np.nan, 2.0], [1.0, np.inf, 2.0], [-np.inf, -np.inf, -np.inf],
                    [-np.inf, 0.0, 1.0]])
    y = oracle.softmax_rows(x)
    assert np.all(np.isnan(y[0])) and np.all(np.isnan(y[1])) and np.all(np.isnan(y[2]))
    ref = _torch_softmax64(np.float64([[-np.inf, 0.0, 1.0]]))[0].astype(np.float32)
    assert np.array_equal(y[3], ref) and y[3][0] == 0.0


def test_strided_rows_leave_padding_untouched():
    rng = np.random.default_rng(6)
    big = rng.standard_normal((9, 40)).astype(np.float32)
    x = big[:, 3:30]                         # ldx = 40, cols = 27
    out_big = np.full((9, 50), 7.0, np.float32)
    out = out_big[:, 5:32]                   # ldy = 50
    oracle.softmax_rows(x, out=out)
    assert np.array_equal(out, oracle.softmax_rows(np.ascontiguousarray(x)))
    pad = np.ones_like(out_big, bool)
    pad[:, 5:32] = False
    assert np.all(out_big[pad] == 7.0)


def test_bf16_rows_are_rounded_fp32_rows():
    rng = np.random.default_rng(7)
    xf = (rng.standard_normal((16, 4096)) * 8).astype(np.float32)
    xb = torch.from_numpy(xf).to(torch.bfloat16)
    xbits = xb.view(torch.int16).numpy().view(np.uint16).copy()
    xbits[:, ::97] = 0xC61C                  # -9984, the masked entries
    y = oracle.softmax_rows(xbits)
    wide = torch.from_numpy(xbits.view(np.int16)).view(torch.bfloat16).float().numpy()
    yf = oracle.softmax_rows(wide)
    ref = torch.from_numpy(yf).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(y, ref)
    assert np.all(y[:, ::97] == 0)           # exp(-9984 - max) is 0


def test_thread_count_does_not_change_bits():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((101, 777)).astype(np.float32)
    a = oracle.softmax_rows(x, threads=1)
    b = oracle.softmax_rows(x, threads=6)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
