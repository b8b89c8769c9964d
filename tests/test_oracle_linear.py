"""Pins for the oracle's Linear + GELU (CPU only).

The product is numpy's float64 matmul (a library primitive used as one
step), so the pins target what could go wrong around it: the orientation
(x w^T, w holding one row per output feature), the bias, the GELU and the
rounding. Checked against a pure-Python triple loop on tiny shapes, torch's
float64 linear + tanh-GELU, the identity and zero weights, and the rounding
chains double -> fp32 -> bf16 and double -> fp32 -> fp16.
"""
import numpy as np
import torch
import torch.nn.functional as F

import oracle

RNG = np.random.default_rng(11)


def test_brute_force_tiny():
    M, N, K = 3, 4, 5
    x = RNG.standard_normal((M, K))
    w = RNG.standard_normal((N, K))
    b = RNG.standard_normal(N)
    want = np.empty((M, N))
    for i in range(M):
        for j in range(N):
            s = b[j]
            for k in range(K):
                s += x[i, k] * w[j, k]
            want[i, j] = s
    got = oracle.linear_gelu(x, w, b, gelu=False)
    assert np.allclose(got, want.astype(np.float32), rtol=1e-6, atol=1e-6)


def test_matches_torch_linear_and_gelu():
    x = RNG.standard_normal((17, 40))
    w = RNG.standard_normal((23, 40)) * 0.2
    b = RNG.standard_normal(23)
    ref = F.gelu(F.linear(torch.from_numpy(x), torch.from_numpy(w), torch.from_numpy(b)),
                 approximate="tanh").numpy()
    got = oracle.linear_gelu(x, w, b, gelu=True)
    assert np.array_equal(got, ref.astype(np.float32)) or np.abs(got - ref).max() < 1e-6


def test_identity_and_zero_weights():
    x = RNG.standard_normal((9, 16)).astype(np.float32)
    b = RNG.standard_normal(16).astype(np.float32)
    eye = np.eye(16, dtype=np.float32)
    want = oracle.gelu_tanh_f64(x.astype(np.float64) + b.astype(np.float64)).reshape(9, 16)
    assert np.array_equal(oracle.linear_gelu(x, eye, b), want.astype(np.float32))
    zero = np.zeros((5, 16), np.float32)
    got = oracle.linear_gelu(x, zero, b[:5])
    assert np.array_equal(got, np.broadcast_to(oracle.gelu_tanh(b[:5]), (9, 5)))


def test_bf16_rounding_chain_and_row_sampling():
    x = oracle.f32_to_bf16(RNG.standard_normal((12, 64)).astype(np.float32))
    w = oracle.f32_to_bf16((RNG.standard_normal((20, 64)) * 0.1).astype(np.float32))
    b = oracle.f32_to_bf16(RNG.standard_normal(20).astype(np.float32))
    full = oracle.linear_gelu(x, w, b)
    assert full.dtype == np.uint16 and full.shape == (12, 20)
    d = oracle.bf16_to_f32(x).astype(np.float64) @ oracle.bf16_to_f32(w).astype(np.float64).T
    d += oracle.bf16_to_f32(b).astype(np.float64)
    want = oracle.f32_to_bf16(oracle.gelu_tanh_f64(d).reshape(d.shape).astype(np.float32))
    assert np.array_equal(full, want.reshape(full.shape))
    rows = np.array([0, 5, 11])
    assert np.array_equal(oracle.linear_gelu(x, w, b, rows=rows), full[rows])
    bound = oracle.linear_abs_bound(x, w, rows=rows)
    assert bound.shape == (3, 20) and np.all(bound >= np.abs(d[rows] - oracle.bf16_to_f32(b)))


def test_fp16_rounding_chain():
    x = RNG.standard_normal((10, 48)).astype(np.float16)
    w = (RNG.standard_normal((14, 48)) * 0.1).astype(np.float16)
    b = RNG.standard_normal(14).astype(np.float16)
    got = oracle.linear_gelu(x, w, b)
    assert got.dtype == np.float16 and got.shape == (10, 14)
    ref = F.gelu(F.linear(*(torch.from_numpy(a.astype(np.float64)) for a in (x, w, b))),
                 approximate="tanh").numpy()
    assert np.array_equal(got, ref.astype(np.float32).astype(np.float16))


def test_relu_epilogue_matches_torch():
    x = RNG.standard_normal((11, 24))
    w = RNG.standard_normal((7, 24))
    b = RNG.standard_normal(7)
    got = oracle.linear_gelu(x, w, b, activation="relu")
    ref = torch.relu(F.linear(torch.from_numpy(x), torch.from_numpy(w), torch.from_numpy(b)))
    assert np.array_equal(got, ref.numpy().astype(np.float32))
    assert np.array_equal(oracle.linear_gelu(x, w, b, activation="none"),
                          oracle.linear_gelu(x, w, b, gelu=False))
