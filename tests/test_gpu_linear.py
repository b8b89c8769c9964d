"""GPU parity of the Linear + GELU kernel (MFMA) against the CPU oracle.
Needs an MI355X.

Tolerance (derived from the arithmetic; none is stated for the
matmul): the kernel accumulates the K products in fp32 in an
order the matrix cores choose, so any summation order must pass:
|y - r| <= ulp_bf16(|r|) + 1.13 (K + 2) 2^-24 ((|x| |w|^T)_ij + |b_j|)
(the rounding of y to bf16, plus the worst-case fp32 accumulation error,
through GELU's slope <= 1.13). As a sharper statistical check, at least
99 % of the outputs must be within one bf16 ulp of the oracle. fp16 data:
the same with the fp16 ulp.
"""
import numpy as np
import pytest
import torch

import memory_bound_elementwise_fk_amd as fk
import oracle
from memory_bound_elementwise_fk_amd import workloads as wl
from tests.gpu_util import DEV, to_dev, to_host

pytestmark = pytest.mark.gpu


def bf16_ulp(r):
    e = np.floor(np.log2(np.maximum(np.abs(r), 2.0 ** -126)))
    return np.exp2(e - 7)


def fp16_ulp(r):
    e = np.floor(np.log2(np.maximum(np.abs(r), 2.0 ** -14)))
    return np.exp2(e - 10)


def f64(a):
    return oracle.bf16_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)


def store(a, dt):
    """float32 values -> the storage of dt (bf16 bits or float16)."""
    a = np.asarray(a, np.float32)
    return a.astype(np.float16) if dt == "fp16" else wl.f32_to_bf16_bits(a).reshape(a.shape)


def operands(M, N, K, seed, bias=True, dt="bf16"):
    rng = np.random.default_rng(seed)
    x = store(rng.standard_normal((M, K)), dt)
    w = store(rng.standard_normal((N, K)) / np.sqrt(max(K, 1)), dt)
    b = store(rng.standard_normal(N), dt) if bias else None
    return x, w, b


def check(got, x, w, b, gelu, what, rows=None):
    ref = oracle.linear_gelu(x, w, b, gelu=gelu, rows=rows)
    g = f64(got)
    r = f64(ref)
    ulp = fp16_ulp if x.dtype == np.float16 else bf16_ulp
    K = x.shape[1]
    scale = oracle.linear_abs_bound(x, w, rows=rows)
    if b is not None:
        scale = scale + np.abs(f64(b))[None, :]
    lim = ulp(r) + 1.13 * (K + 2) * 2.0 ** -24 * scale
    err = np.abs(g - r)
    bad = np.flatnonzero(err > lim)
    assert bad.size == 0, f"{what}: {bad.size} beyond the bound, worst excess {(err - lim).max():.3e}"
    within = np.mean(err <= ulp(r))
    assert within >= 0.99, f"{what}: only {within:.4f} of outputs within one bf16 ulp"


# K % 64 == 0 takes the direct-to-LDS kernel with K steps of 64, other
# K % 32 == 0 the one with K steps of 32 (rows past M or N clamped in both),
# other K the register-staged one
@pytest.mark.parametrize("M,N,K", [(1, 1, 8), (7, 13, 24), (300, 200, 392), (256, 256, 64),
                                   (257, 511, 520), (512, 768, 1024), (1000, 300, 8),
                                   (1, 1, 32), (33, 65, 96), (300, 200, 384), (257, 511, 1024),
                                   (513, 257, 4096)])
@pytest.mark.parametrize("gelu", [True, False])
@pytest.mark.parametrize("dt", ["bf16", "fp16"])
def test_linear_shapes(M, N, K, gelu, dt):
    x, w, b = operands(M, N, K, seed=M * 7 + N + K, dt=dt)
    y = fk.linear_gelu(to_dev(x), to_dev(w), to_dev(b), gelu=gelu)
    check(to_host(y), x, w, b, gelu, f"{dt} {M}x{N}x{K} gelu={gelu}")


@pytest.mark.parametrize("M,N,K", [(300, 200, 392), (257, 511, 1024)])  # both main loops
@pytest.mark.parametrize("dt", ["bf16", "fp16"])
def test_linear_relu_epilogue(M, N, K, dt):
    x, w, b = operands(M, N, K, seed=M + N + K + 1, dt=dt)
    y = fk.linear_gelu(to_dev(x), to_dev(w), to_dev(b), activation="relu")
    got = to_host(y)
    ref = oracle.linear_gelu(x, w, b, activation="relu")
    g, r = f64(got), f64(ref)
    ulp = fp16_ulp if dt == "fp16" else bf16_ulp
    scale = oracle.linear_abs_bound(x, w) + np.abs(f64(b))[None, :]
    assert np.all(np.abs(g - r) <= ulp(r) + (K + 2) * 2.0 ** -24 * scale), f"relu {dt} {M}x{N}x{K}"
    assert np.all(g >= 0) and not np.any(np.signbit(g)), "ReLU output must be +0 or positive"


def test_linear_without_bias_and_k_zero():
    x, w, _ = operands(130, 70, 40, seed=3, bias=False)
    y = fk.linear_gelu(to_dev(x), to_dev(w), None)
    check(to_host(y), x, w, None, True, "no bias")
    # K == 0: the product is empty, y = GELU(bias)
    b = wl.f32_to_bf16_bits(np.linspace(-3, 3, 70).astype(np.float32))
    xe = torch.empty((5, 0), dtype=torch.bfloat16, device=DEV)
    we = torch.empty((70, 0), dtype=torch.bfloat16, device=DEV)
    ye = fk.linear_gelu(xe, we, to_dev(b))
    assert np.array_equal(to_host(ye), np.broadcast_to(oracle.gelu_tanh(b), (5, 70)))


@pytest.mark.parametrize("K", [136, 160, 192])  # register-staged / direct (32) / direct (64)
def test_linear_strided_operands(K):
    M, N = 300, 260
    x, w, b = operands(M, N, K, seed=5)
    xb = np.zeros((M, K + 8), np.uint16)
    xb[:, :K] = x
    wb = np.zeros((N, K + 16), np.uint16)
    wb[:, :K] = w
    ybuf = torch.full((M, N + 3), 0x7FC1, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    fk.fk_linear_gelu(to_dev(xb)[:, :K], to_dev(wb)[:, :K], to_dev(b), ybuf[:, :N])
    got = to_host(ybuf)
    check(got[:, :N], x, w, b, True, "strided")
    assert np.all(got[:, N:] == 0x7FC1), "row padding of y was written"


@pytest.mark.parametrize("dt", ["bf16", "fp16"])
def test_linear_mlp_shape_sampled_rows(dt):
    # the MLP up-projection shape the bench times: 8192 x 4096 -> 16384
    M, N, K = 8192, 16384, 4096
    x, w, b = operands(M, N, K, seed=9, dt=dt)
    y = fk.linear_gelu(to_dev(x), to_dev(w), to_dev(b))
    rows = np.sort(np.random.default_rng(10).choice(M, 48, replace=False))
    got = to_host(y[torch.from_numpy(rows).to(DEV)])
    check(got, x, w, b, True, f"{dt} 8192x16384x4096 sampled rows", rows=rows)


@pytest.mark.parametrize("dt", ["bf16", "fp16"])
def test_linear_unaligned_bias_and_output(dt):
    # bias one element past an aligned address and an output row stride that
    # is not a multiple of 4, with M and N ragged against the 256 x 256 tiles
    M, N, K = 300, 270, 128
    x, w, b = operands(M, N, K, seed=21, dt=dt)
    bpad = np.zeros(N + 1, b.dtype)
    bpad[1:] = b
    bdev = to_dev(bpad)[1:]
    assert bdev.data_ptr() % 8 != 0
    tdt = torch.float16 if dt == "fp16" else torch.bfloat16
    ybuf = torch.full((M, N + 1), 0x7FC1 if dt == "bf16" else 0x7E01, dtype=torch.int16,
                      device=DEV).view(tdt)
    fk.fk_linear_gelu(to_dev(x), to_dev(w), bdev, ybuf[:, :N])
    got = to_host(ybuf)
    check(got[:, :N], x, w, b, True, f"{dt} unaligned bias/output")
    pad = np.ascontiguousarray(got[:, N:]).view(np.uint16)
    assert np.all(pad == (0x7FC1 if dt == "bf16" else 0x7E01)), "row padding of y was written"


def test_linear_is_bitwise_reproducible():
    x, w, b = operands(512, 512, 512, seed=12)
    xt, wt, bt = to_dev(x), to_dev(w), to_dev(b)
    a = fk.linear_gelu(xt, wt, bt)
    c = fk.linear_gelu(xt, wt, bt)
    assert torch.equal(a.view(torch.int16), c.view(torch.int16))
