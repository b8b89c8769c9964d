"""Pins for the oracle's attention forward (CPU only).

The oracle is the plain definition O = softmax(Q K^T / sqrt(d) + mask) V
(FlashAttention computes exactly this, tile by tile, in "Lecture 6: GPU
Kernels and Triton", sections 7.3 and 8; the causal mask keeps key j <= i).
Pinned against torch's scaled_dot_product_attention in float64, and by
cases with closed forms: Q = 0 gives uniform weights (O = mean of the
allowed V rows: the prefix mean under the causal mask), one dominant score
selects its V row, T = 1 and the first causal row give V[0], and without
the mask a joint permutation of K and V leaves O unchanged. bf16 and fp16
data are the double result rounded to fp32 and then to the storage type.
"""
import numpy as np
import torch
import torch.nn.functional as F

import oracle

RNG = np.random.default_rng(21)


def test_matches_torch_sdpa():
    for causal in (True, False):
        q, k, v = (RNG.standard_normal((2, 3, 37, 16)) for _ in range(3))
        ref = F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k),
                                             torch.from_numpy(v), is_causal=causal).numpy()
        got = oracle.attention(q.astype(np.float32), k.astype(np.float32), v.astype(np.float32),
                               causal=causal)
        # inputs were rounded to fp32 for the oracle: compare at that precision
        ref32 = F.scaled_dot_product_attention(
            torch.from_numpy(q.astype(np.float32).astype(np.float64)),
            torch.from_numpy(k.astype(np.float32).astype(np.float64)),
            torch.from_numpy(v.astype(np.float32).astype(np.float64)), is_causal=causal).numpy()
        assert np.abs(got - ref32).max() < 1e-6
        assert np.abs(got - ref).max() < 1e-5


def test_zero_queries_give_prefix_means():
    T, d = 20, 8
    q = np.zeros((1, 1, T, d), np.float32)
    k = RNG.standard_normal((1, 1, T, d)).astype(np.float32)
    v = RNG.standard_normal((1, 1, T, d)).astype(np.float32)
    causal = oracle.attention(q, k, v, causal=True)[0, 0]
    prefix = np.cumsum(v[0, 0].astype(np.float64), axis=0) / np.arange(1, T + 1)[:, None]
    assert np.abs(causal - prefix).max() < 1e-6
    full = oracle.attention(q, k, v, causal=False)[0, 0]
    assert np.abs(full - v[0, 0].astype(np.float64).mean(axis=0)).max() < 1e-6


def test_dominant_score_selects_its_value_row():
    T, d = 12, 4
    k = RNG.standard_normal((1, 1, T, d)).astype(np.float32)
    v = RNG.standard_normal((1, 1, T, d)).astype(np.float32)
    q = np.zeros((1, 1, T, d), np.float32)
    q[0, 0, :, 0] = 300.0
    k[0, 0, :, 0] = 0.0
    k[0, 0, 5, 0] = 1.0                     # key 5 scores 150, the others 0
    o = oracle.attention(q, k, v, causal=False)[0, 0]
    assert np.allclose(o, np.broadcast_to(v[0, 0, 5], (T, d)), atol=1e-6)


def test_single_position_and_first_causal_row():
    q, k, v = (RNG.standard_normal((1, 2, 1, 8)).astype(np.float32) for _ in range(3))
    assert np.array_equal(oracle.attention(q, k, v), v)
    q, k, v = (RNG.standard_normal((1, 1, 9, 8)).astype(np.float32) for _ in range(3))
    assert np.array_equal(oracle.attention(q, k, v, causal=True)[0, 0, 0], v[0, 0, 0])


def test_joint_permutation_of_keys_and_values():
    q, k, v = (RNG.standard_normal((1, 1, 15, 8)).astype(np.float32) for _ in range(3))
    perm = RNG.permutation(15)
    a = oracle.attention(q, k, v, causal=False)
    b = oracle.attention(q, k[:, :, perm], v[:, :, perm], causal=False)
    assert np.abs(a - b).max() < 1e-6


def test_bf16_rounding_and_sampled_rows():
    q, k, v = (oracle.f32_to_bf16(RNG.standard_normal((1, 2, 33, 16)).astype(np.float32))
               .reshape(1, 2, 33, 16) for _ in range(3))
    full = oracle.attention(q, k, v)
    assert full.dtype == np.uint16
    part = oracle.attention(q, k, v, rows={(0, 1): np.array([0, 7, 32])})
    assert np.array_equal(part[(0, 1)], full[0, 1][[0, 7, 32]])


def test_fp16_data_round_the_double_result_twice():
    """fp16 inputs: the double result rounded to fp32, then to fp16 (nearest
    even, numpy's conversion), pinned against torch SDPA in float64 on the
    same fp16 values; within one fp16 ulp of the double result."""
    q, k, v = (RNG.standard_normal((1, 2, 40, 32)).astype(np.float16) for _ in range(3))
    for causal in (True, False):
        got = oracle.attention(q, k, v, causal=causal)
        assert got.dtype == np.float16
        ref = F.scaled_dot_product_attention(
            *(torch.from_numpy(a.astype(np.float64)) for a in (q, k, v)), is_causal=causal).numpy()
        assert np.array_equal(got, ref.astype(np.float32).astype(np.float16))
        ulp = np.spacing(np.abs(ref).astype(np.float16)).astype(np.float64)
        assert np.all(np.abs(got.astype(np.float64) - ref) <= ulp)
    part = oracle.attention(q, k, v, rows={(0, 1): np.array([0, 39])})
    assert np.array_equal(part[(0, 1)], oracle.attention(q, k, v)[0, 1][[0, 39]])
