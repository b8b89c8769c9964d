"""GPU parity of the backward kernels (GELU and row softmax) against the CPU
oracle. Needs an MI355X.

Tolerances (derived from the kernels' fp32 arithmetic; the pages state none
for backward passes):
  * GELU backward, fp32: |dx - r| <= 1e-5 |r| + 2e-6 |dy| + FLT_MIN. GELU'
    is s + w s q with both terms up to ~0.5 in magnitude for |x| < 3 and a
    zero crossing near x = -0.75 (GELU's minimum), where the sum cancels:
    there the absolute rounding of the terms (a few 2^-24, plus the exponent
    argument's ~2^-21 relative for |t| up to ~25) bounds the error, times
    |dy|. bf16: one bf16 ulp of r plus the same absolute term.
  * Softmax backward, fp32: |dx_j - r_j| <= 2e-6 max_row|dy|: the row dot
    product is a tree sum with error <= (log2(cols) + 2) 2^-24 max|dy| (the
    y sum to 1), multiplied by y_j <= 1, plus the rounding of the result.
    bf16: one bf16 ulp plus the same absolute term (dy_j - dot can cancel).
"""
import numpy as np
import pytest
import torch

import memory_bound_elementwise_fk_amd as fk
import oracle
from memory_bound_elementwise_fk_amd import workloads as wl
from tests.gpu_util import CANARY_BITS, DEV, guarded, guards_intact, random_input, tdtype, \
    to_dev, to_host

pytestmark = pytest.mark.gpu
T = oracle.default_threads()
FLT_MIN = float(np.finfo(np.float32).tiny)


def as64(a, dt):
    return (a if dt == "f32" else oracle.bf16_to_f32(a)).astype(np.float64)


def bf16_ulp(r):
    e = np.floor(np.log2(np.maximum(np.abs(r), 2.0 ** -126)))
    return np.exp2(e - 7)


def check(got, ref, dt, abs_term, rel, what):
    g, r = as64(got, dt), as64(ref, dt)
    assert np.array_equal(np.isnan(g), np.isnan(r)), f"{what}: NaN pattern"
    ok = ~np.isnan(r)
    inf = np.isinf(r) & ok
    assert np.array_equal(g[inf], r[inf]), f"{what}: infinities"
    ok &= ~inf
    err = np.abs(g[ok] - r[ok])
    lim = np.broadcast_to(abs_term, r.shape)[ok] + (rel * np.abs(r[ok]) if dt == "f32"
                                                   else bf16_ulp(r[ok]))
    bad = np.flatnonzero(err > lim)
    assert bad.size == 0, f"{what}: {bad.size} beyond tolerance, worst excess {(err - lim).max():.3e}"


def gelu_bwd_check(x, dy, dt, what, dx=None):
    ref = oracle.gelu_tanh_backward(x, dy, threads=T)
    if dx is None:
        xt, dyt = to_dev(x), to_dev(dy)
        full, dxt = guarded(x.shape, tdtype(dt))
        fk.fk_gelu_tanh_backward(xt, dyt, dxt)
        dx = to_host(dxt)
        assert guards_intact(full, x.size), "wrote outside dx"
    check(dx, ref, dt, 2e-6 * np.abs(as64(dy, dt)) + FLT_MIN, 1e-5, what)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("n", [1, 3, 7, 8, 9, 63, 64, 65, 511, 512, 513, 4097, 100_003, 1 << 20])
def test_gelu_backward_ragged_sizes(dt, n):
    x = random_input((n,), dt, 3.0, seed=n)
    dy = random_input((n,), dt, 1.0, seed=n + 1)
    gelu_bwd_check(x, dy, dt, f"gelu bwd {dt} n={n}")


def test_gelu_backward_fp32_dense_sweep_and_tail():
    lo, hi = np.float32(-9.5).view(np.uint32), np.float32(12.0).view(np.uint32)
    neg = np.arange(np.uint32(0x80000000), lo, 61, dtype=np.uint32).view(np.float32)
    pos = np.arange(0, hi, 61, dtype=np.uint32).view(np.float32)
    tail = -np.geomspace(9.5, 40.0, 100_001).astype(np.float32)
    x = np.concatenate([neg, pos, tail])
    dy = np.random.default_rng(3).standard_normal(x.size).astype(np.float32)
    gelu_bwd_check(x, dy, "f32", "dense sweep")


def test_gelu_backward_special_values():
    x = np.float32([0.0, -0.0, np.inf, -np.inf, np.nan, 12.0, 1e20, -1e20, 3e38, -3e38, -0.7518])
    dy = np.float32([2.0, 2.0, 3.0, 3.0, 1.0, 1.0, 1.0, 1.0, 1.0, 1.0, 1.0])
    xt, dyt = to_dev(x), to_dev(dy)
    dx = fk.gelu_tanh_backward(xt, dyt)
    got = to_host(dx)
    gelu_bwd_check(x, dy, "f32", "specials", dx=got)
    assert got[0] == 1.0 and got[1] == 1.0               # GELU'(0) = 1/2
    assert got[2] == 3.0 and got[3] == 0.0               # limits 1 and 0
    assert np.isnan(got[4])
    assert np.all(got[5:7] == 1.0)                      # x = 12, 1e20
    assert got[7] == 0.0 and got[8] == 1.0 and got[9] == 0.0   # -1e20, 3e38, -3e38


def test_gelu_backward_every_bf16_pattern():
    x = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    dy = wl.f32_to_bf16_bits(np.random.default_rng(4).standard_normal(1 << 16).astype(np.float32))
    gelu_bwd_check(x, dy, "bf16", "all bf16 x")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_gelu_backward_in_place_and_unaligned(dt):
    n = 50_001
    x = random_input((n + 2,), dt, 2.0, seed=5)
    dy = random_input((n + 2,), dt, 1.0, seed=6)
    ref = oracle.gelu_tanh_backward(x[:n], dy[:n])
    xt, dyt = to_dev(x[:n]), to_dev(dy[:n])
    fk.fk_gelu_tanh_backward(xt, dyt, dyt)                 # dx == dy
    check(to_host(dyt), ref, dt, 2e-6 * np.abs(as64(dy[:n], dt)) + FLT_MIN, 1e-5, "dx == dy")
    xt2, dyt2 = to_dev(x[:n]), to_dev(dy[:n])
    fk.fk_gelu_tanh_backward(xt2, dyt2, xt2)               # dx == x
    check(to_host(xt2), ref, dt, 2e-6 * np.abs(as64(dy[:n], dt)) + FLT_MIN, 1e-5, "dx == x")
    xu, dyu = to_dev(x)[1:n + 1], to_dev(dy)[2:n + 2]     # misaligned operands
    dxu = torch.empty(n + 1, dtype=tdtype(dt), device=DEV)[1:]
    fk.fk_gelu_tanh_backward(xu, dyu, dxu)
    ref_u = oracle.gelu_tanh_backward(x[1:n + 1], dy[2:n + 2])
    check(to_host(dxu), ref_u, dt, 2e-6 * np.abs(as64(dy[2:n + 2], dt)) + FLT_MIN, 1e-5,
          "unaligned")


def test_gelu_backward_bf16_large():
    n = 1 << 26
    x = wl.draw(n, seed=0, dtype="bf16")
    dy = wl.draw(n, seed=0, stream=1, dtype="bf16")
    gelu_bwd_check(x, dy, "bf16", "bf16 2^26")


def test_gelu_backward_bf16_beyond_one_launch_grid():
    # 2^34 + 1001 bf16 elements (32 GiB per tensor, x, dy and dx: 96 GiB):
    # more tiles than one launch's 2^31 work-items, so the kernel strides
    # over tiles; checked on sampled outputs (random, first tiles, ragged tail)
    n = (1 << 34) + 1001
    gen = torch.Generator(device=DEV)
    gen.manual_seed(7)
    x = torch.randn(n, dtype=torch.bfloat16, device=DEV, generator=gen).mul_(3)
    dy = torch.randn(n, dtype=torch.bfloat16, device=DEV, generator=gen)
    dx = torch.empty_like(x)
    fk.fk_gelu_tanh_backward(x, dy, dx)
    rng = np.random.default_rng(8)
    idx = np.unique(np.concatenate([rng.integers(0, n, 1 << 20), np.arange(5000),
                                    np.arange(n - 5000, n)]))
    it = torch.from_numpy(idx).to(DEV)
    xs, dys, dxs = (wl.from_torch(t[it]) for t in (x, dy, dx))
    del x, dy, dx
    torch.cuda.empty_cache()
    gelu_bwd_check(xs, dys, "bf16", "bf16 2^34 + 1001, sampled", dx=dxs)


# ---------------------------------------------------------- softmax bwd ---
def softmax_pair(rows, cols, dt, seed, scale=3.0):
    x = random_input((rows, cols), dt, scale, seed=seed)
    y = oracle.softmax_rows(x, threads=T)
    dy = random_input((rows, cols), dt, 1.0, seed=seed + 1)
    return y, dy


def sbwd_check(got, y, dy, dt, what):
    ref = oracle.softmax_rows_backward(y, dy, threads=T)
    dmax = np.abs(as64(dy, dt)).max(axis=1, keepdims=True)
    check(got, ref, dt, 2e-6 * dmax, 2e-6, what)


def run_sbwd(y, dy, dt):
    yt, dyt = to_dev(y), to_dev(dy)
    full, dx = guarded(y.shape, tdtype(dt))
    fk.fk_softmax_rows_backward(yt, dyt, dx)
    got = to_host(dx)
    assert guards_intact(full, y.size), "wrote outside dx"
    return got


# ragged widths; widths that fill a row shape exactly (the unmasked kernel
# variant, also of the 3-, 5-, 6- and 12-wave shapes) for both dtypes;
# multiples of the vector inside a shape (the per-vector masks)
SCOLS = [1, 2, 3, 63, 64, 65, 256, 512, 1000, 1023, 1024, 1025, 1536, 2048, 2560, 3000, 3072,
         4096, 4097, 5000, 5120, 6144, 8192, 10240, 12000, 12288, 16384, 16385, 24576, 32768]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("cols", SCOLS)
def test_softmax_backward_widths(dt, cols):
    if cols > fk.fk_softmax_backward_max_cols(tdtype(dt)):
        # wider than the kernel's capacity for this dtype: refused before any
        # launch, dx keeps its contents
        y, dy = (to_dev(random_input((2, cols), dt, 1.0, seed=cols + k)) for k in (0, 1))
        dx = torch.zeros_like(y)
        with pytest.raises(fk.FusedOpsError) as err:
            fk.fk_softmax_rows_backward(y, dy, dx)
        assert err.value.status == fk.FK_ERR_UNSUPPORTED
        assert not bool(dx.view(torch.int16 if dt == "bf16" else torch.int32).any())
        return
    rows = 3 if cols > 4096 else 17
    y, dy = softmax_pair(rows, cols, dt, cols)
    sbwd_check(run_sbwd(y, dy, dt), y, dy, dt, f"softmax bwd {dt} cols={cols}")


def test_softmax_backward_c4_shape_bf16():
    x = wl.make_input("C4")
    y = oracle.softmax_rows(x, threads=T)
    dy = wl.draw(x.size, seed=0, stream=2, dtype="bf16").reshape(x.shape)
    yt, dyt = to_dev(y), to_dev(dy)
    dx = torch.empty_like(yt)
    fk.fk_softmax_rows_backward(yt, dyt, dx)
    got = to_host(dx)
    del yt, dyt, dx
    sbwd_check(got, y, dy, "bf16", "C4 shape")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_softmax_backward_strided_in_place_unaligned(dt):
    rows, cols, ld = 7, 1000, 1008
    y, dy = softmax_pair(rows, cols, dt, 91)
    ypad = np.zeros((rows, ld), y.dtype)
    ypad[:, :cols] = y
    yt = to_dev(ypad)[:, :cols]
    full, dxbig = guarded((rows, ld), tdtype(dt))
    fk.fk_softmax_rows_backward(yt, to_dev(dy), dxbig[:, :cols])
    got = to_host(dxbig)
    assert guards_intact(full, rows * ld)
    sbwd_check(got[:, :cols], y, dy, dt, "strided")
    assert np.all(got[:, cols:].view(np.uint16 if dt == "bf16" else np.uint32) == CANARY_BITS[dt])
    dyt = to_dev(dy)
    fk.fk_softmax_rows_backward(to_dev(y), dyt, dyt)       # dx == dy
    sbwd_check(to_host(dyt), y, dy, dt, "in place")
    flat_y = np.concatenate([y.ravel()[:1], y.ravel()])
    yu = to_dev(flat_y)[1:].view(rows, cols)               # misaligned: scalar path
    dxu = torch.empty(rows * cols + 1, dtype=tdtype(dt), device=DEV)[1:].view(rows, cols)
    fk.fk_softmax_rows_backward(yu, to_dev(dy), dxu)
    sbwd_check(to_host(dxu), y, dy, dt, "unaligned")


def test_softmax_backward_identities():
    rows, cols = 6, 2000
    y, dy = softmax_pair(rows, cols, "f32", 93)
    got = run_sbwd(y, dy, "f32")
    assert np.abs(got.astype(np.float64).sum(axis=1)).max() < 1e-5     # rows of dx sum to ~0
    onehot = np.zeros((rows, cols), np.float32)
    onehot[np.arange(rows), np.arange(rows) * 7] = 1.0
    assert np.all(run_sbwd(onehot, dy, "f32") == 0)                    # exactly zero
    const = run_sbwd(y, np.full((rows, cols), 0.75, np.float32), "f32")
    assert np.abs(const).max() <= 2e-6


def test_softmax_backward_rows_beyond_one_launch_grid():
    # 2^25 + 5 rows of 3 fp32 columns: the kernel strides over rows
    rows, cols = (1 << 25) + 5, 3
    gen = torch.Generator(device=DEV)
    gen.manual_seed(21)
    y = torch.softmax(torch.randn(rows, cols, device=DEV, generator=gen) * 2, dim=1)
    dy = torch.randn(rows, cols, device=DEV, generator=gen)
    dx = fk.softmax_rows_backward(y, dy)
    rng = np.random.default_rng(22)
    idx = np.unique(np.concatenate([rng.integers(0, rows, 200_000), np.arange(rows - 100, rows)]))
    it = torch.from_numpy(idx).to(DEV)
    ys, dys, dxs = (wl.from_torch(t[it]) for t in (y, dy, dx))
    del y, dy, dx
    torch.cuda.empty_cache()
    sbwd_check(dxs, ys, dys, "f32", f"softmax backward {rows}x{cols}, sampled rows")
