"""GPU parity of the fused LayerNorm (+ optional tanh-GELU) row kernel against
the CPU oracle. Needs an MI355X.

Tolerances (none is stated for LayerNorm; derived from the fp32
arithmetic of the kernel):
  * fp32: |y - r| <= 4e-6 |r| + atol, atol = 4 (log2(cols) + 2) 2^-24 max|gamma|
    + 2^-24 max|beta|. The relative part covers the rounding of var, rstd and
    the final products (a few ulps); the absolute part bounds the error of
    the corrected mean (tree summation of the deviations, log2(cols) + 2
    roundings of magnitude ~2^-24 sigma, times rstd ~ 1/sigma), which enters
    every output times gamma, plus the rounding of beta. With the GELU
    epilogue, add GELU's own 1e-5 relative (its slope is below 1.13).
  * bf16: |y - r| <= ulp_bf16(|r|) + atol + rtol |r| with atol, rtol as above
    (y, r the bf16 results as numbers): the fp32 error can move the value
    before both sides round to bf16, half an ulp each. Far from zero this is
    one bf16 ulp; where gamma * t + beta cancels to a value near zero the
    fp32 absolute error dominates, and no fp32 schedule can promise one ulp
    of that small result.
"""
import math

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


def params(cols, dt, seed, affine=True):
    if not affine:
        return None, None
    rng = np.random.default_rng(seed)
    g = (1.0 + 0.25 * rng.standard_normal(cols)).astype(np.float32)
    b = (0.5 * rng.standard_normal(cols)).astype(np.float32)
    if dt == "bf16":
        g, b = wl.f32_to_bf16_bits(g), wl.f32_to_bf16_bits(b)
    return g, b


def as_f32(a, dt):
    return a if dt == "f32" else oracle.bf16_to_f32(a)


def bf16_ulp(r):
    """Spacing of bf16 values at |r| (2^(e - 7) for a normal r, 2^-133 below)."""
    e = np.floor(np.log2(np.maximum(np.abs(r), 2.0 ** -126)))
    return np.exp2(e - 7)


def assert_ln(got, ref, dt, cols, g, b, gelu, what):
    gmax = 1.0 if g is None else float(np.abs(g).max())
    bmax = 0.0 if b is None else float(np.abs(b).max())
    atol = 4 * (math.log2(max(cols, 1)) + 2) * 2.0 ** -24 * gmax + 2.0 ** -24 * bmax
    rtol = 4e-6 + (1e-5 if gelu else 0.0)
    if dt == "bf16":
        g64 = oracle.bf16_to_f32(got).astype(np.float64)
        r64 = oracle.bf16_to_f32(ref).astype(np.float64)
        assert np.array_equal(np.isnan(g64), np.isnan(r64)), f"{what}: NaN pattern"
        ok = ~np.isnan(r64)
        err = np.abs(g64[ok] - r64[ok])
        lim = bf16_ulp(r64[ok]) + atol + rtol * np.abs(r64[ok])
        bad = np.flatnonzero(err > lim)
        assert bad.size == 0, f"{what}: {bad.size} beyond tolerance, worst excess {(err - lim).max():.3e}"
        return
    g64, r64 = got.astype(np.float64), ref.astype(np.float64)
    assert np.array_equal(np.isnan(g64), np.isnan(r64)), f"{what}: NaN pattern"
    ok = ~np.isnan(r64)
    err = np.abs(g64[ok] - r64[ok])
    lim = rtol * np.abs(r64[ok]) + atol
    bad = np.flatnonzero(err > lim)
    assert bad.size == 0, f"{what}: {bad.size} beyond tolerance, worst excess {(err - lim).max():.3e}"


def run(x, dt, g=None, b=None, gelu=False, eps=1e-5):
    xt = to_dev(x)
    full, y = guarded(x.shape, tdtype(dt))
    gt = None if g is None else to_dev(g)
    bt = None if b is None else to_dev(b)
    fk.fk_layernorm_rows(xt, y, gt, bt, eps=eps, gelu=gelu)
    got = to_host(y)
    assert guards_intact(full, x.size), "layernorm wrote outside its output"
    return got


# ragged widths; widths that fill a row shape exactly (256 * 2^k, and 768 ...
# 24576 for the 3-, 5-, 6-, 10- and 12-wave shapes: the unmasked kernel
# variant) for both dtypes; multiples of the vector inside a shape (1000,
# 3000, 5000, 12000: the per-vector masks)
COLS = [1, 2, 3, 63, 64, 65, 255, 256, 512, 768, 1000, 1023, 1024, 1025, 1280, 1536, 2048, 2560,
        3000, 3072, 4095, 4096, 4097, 5000, 5120, 6144, 8192, 8193, 10240, 12000, 12288, 16384,
        24576, 32768, 65536]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("cols", COLS)
def test_layernorm_widths(dt, cols):
    if cols > fk.fk_layernorm_max_cols(tdtype(dt)):
        # wider than the kernel's capacity for this dtype: refused before any
        # launch, y keeps its contents
        x = to_dev(random_input((2, cols), dt, 1.0, seed=cols))
        y = torch.zeros_like(x)
        with pytest.raises(fk.FusedOpsError) as err:
            fk.fk_layernorm_rows(x, y)
        assert err.value.status == fk.FK_ERR_UNSUPPORTED
        assert not bool(y.view(torch.int16 if dt == "bf16" else torch.int32).any())
        return
    rows = 3 if cols > 8192 else 13
    x = random_input((rows, cols), dt, 3.0, seed=cols)
    if dt == "f32":
        x = x + np.float32(20.0) * (np.arange(rows, dtype=np.float32)[:, None] % 3)
    g, b = params(cols, dt, cols + 1)
    for gelu in (False, True):
        ref = oracle.layernorm_rows(x, g, b, gelu=gelu)
        assert_ln(run(x, dt, g, b, gelu), ref, dt, cols, as_f32(g, dt), as_f32(b, dt), gelu,
                  f"{dt} cols={cols} gelu={gelu}")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("cols", [777, 1024])
def test_layernorm_without_affine_and_eps(dt, cols):
    x = random_input((33, cols), dt, 0.01, seed=5)
    for eps in (0.0, 1e-5, 0.1):
        ref = oracle.layernorm_rows(x, eps=eps)
        assert_ln(run(x, dt, eps=eps), ref, dt, cols, None, None, False, f"no affine eps={eps}")
    g, b = params(cols, dt, 6)
    ref = oracle.layernorm_rows(x, g, None)
    assert_ln(run(x, dt, g, None), ref, dt, cols, as_f32(g, dt), None, False, "gamma only")
    ref = oracle.layernorm_rows(x, None, b, gelu=True)
    assert_ln(run(x, dt, None, b, gelu=True), ref, dt, cols, None, as_f32(b, dt), True,
              "beta only")


def test_ln1_full_size_fp32_shifted_rows():
    # C2's rows: 4096 x 1000, x ~ N(0, 3^2), every 16th row shifted by +80
    x = wl.make_input("C2")
    g, b = params(1000, "f32", 7)
    ref = oracle.layernorm_rows(x, g, b, threads=T)
    got = run(x, "f32", g, b)
    assert_ln(got, ref, "f32", 1000, g, b, False, "LN fp32 4096x1000")
    ref_g = oracle.layernorm_rows(x, g, b, gelu=True, threads=T)
    assert_ln(run(x, "f32", g, b, True), ref_g, "f32", 1000, g, b, True, "LN+GELU fp32")


def test_ln2_full_size_bf16():
    # C4's shape: 32768 x 4096 bf16, x ~ 8 N(0, 1)
    x = wl.draw(32768 * 4096, seed=0, scale=8.0, dtype="bf16").reshape(32768, 4096)
    g, b = params(4096, "bf16", 8)
    xt = to_dev(x)
    y = torch.empty_like(xt)
    fk.fk_layernorm_rows(xt, y, to_dev(g), to_dev(b), gelu=True)
    got = to_host(y)
    del xt, y
    assert_ln(got, oracle.layernorm_rows(x, g, b, gelu=True, threads=T), "bf16", 4096,
              oracle.bf16_to_f32(g), oracle.bf16_to_f32(b), True, "LN+GELU bf16")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_layernorm_strided_unaligned_in_place(dt):
    rows, cols, ld = 9, 1000, 1016
    xbig = random_input((rows, ld), dt, 2.0, seed=11)
    g, b = params(cols, dt, 12)
    ref = oracle.layernorm_rows(np.ascontiguousarray(xbig[:, :cols]), g, b)
    xt = to_dev(xbig)[:, :cols]
    full, ybig = guarded((rows, ld), tdtype(dt))
    fk.fk_layernorm_rows(xt, ybig[:, :cols], to_dev(g), to_dev(b))
    got = to_host(ybig)
    assert guards_intact(full, rows * ld)
    assert_ln(got[:, :cols], ref, dt, cols, as_f32(g, dt), as_f32(b, dt), False, "strided")
    assert np.all(got[:, cols:].view(np.uint16 if dt == "bf16" else np.uint32) == CANARY_BITS[dt])
    # unaligned rows and parameters (scalar path)
    flat = random_input((rows * cols + 1,), dt, 2.0, seed=13)
    xu = to_dev(flat)[1:].view(rows, cols)
    gu = to_dev(np.concatenate([g[:1], g]))[1:]
    yu = torch.empty(rows * cols + 1, dtype=tdtype(dt), device=DEV)[1:].view(rows, cols)
    fk.fk_layernorm_rows(xu, yu, gu, to_dev(b))
    assert_ln(to_host(yu), oracle.layernorm_rows(flat[1:].reshape(rows, cols), g, b), dt, cols,
              as_f32(g, dt), as_f32(b, dt), False, "unaligned")
    # in place
    xi = to_dev(np.ascontiguousarray(xbig[:, :cols]))
    fk.fk_layernorm_rows(xi, xi, to_dev(g), to_dev(b))
    assert_ln(to_host(xi), ref, dt, cols, as_f32(g, dt), as_f32(b, dt), False, "in place")


def test_layernorm_special_rows():
    cols = 1000
    x = np.random.default_rng(3).standard_normal((4, cols)).astype(np.float32)
    x[0, :] = 2.5                       # constant row: output is beta exactly
    x[1, 17] = np.nan                   # NaN anywhere -> whole row NaN
    x[2, :] = 1e4 + x[2, :]             # far from zero: the corrected mean keeps accuracy
    g, b = params(cols, "f32", 14)
    got = run(x, "f32", g, b)
    ref = oracle.layernorm_rows(x, g, b)
    assert np.array_equal(got[0], b)
    assert np.all(np.isnan(got[1]))
    assert_ln(got[2:], ref[2:], "f32", cols, g, b, False, "specials")


def test_layernorm_bitwise_reproducible():
    x = to_dev(random_input((500, 4096), "bf16", 4.0, seed=15))
    a = fk.layernorm_rows(x, gelu=True)
    c = fk.layernorm_rows(x, gelu=True)
    assert torch.equal(a.view(torch.int16), c.view(torch.int16))


@pytest.mark.parametrize("cols", [1, 3])
def test_layernorm_rows_beyond_one_launch_grid(cols):
    # 2^25 + 5 rows of 1 or 3 fp32 columns: the kernel strides over rows
    rows = (1 << 25) + 5
    gen = torch.Generator(device=DEV)
    gen.manual_seed(cols + 10)
    x = torch.randn(rows, cols, dtype=torch.float32, device=DEV, generator=gen).mul_(3)
    g, b = params(cols, "f32", cols)
    y = fk.layernorm_rows(x, to_dev(g), to_dev(b), gelu=True)
    rng = np.random.default_rng(cols + 10)
    idx = np.unique(np.concatenate([rng.integers(0, rows, 200_000), np.arange(rows - 100, rows)]))
    it = torch.from_numpy(idx).to(DEV)
    xs, ys = wl.from_torch(x[it]), wl.from_torch(y[it])
    del x, y
    torch.cuda.empty_cache()
    assert_ln(ys, oracle.layernorm_rows(xs, g, b, gelu=True), "f32", cols, g, b, True,
              f"layernorm {rows}x{cols}, sampled rows")


# More row groups than the launch's workgroup cap: each workgroup strides
# over many rows (several rows per workgroup on narrow shapes), alternating
# its reduction slots; odd row counts leave a partial last step.
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("cols", [64, 1000])
def test_layernorm_many_rows_grid_strided(dt, cols):
    rows = 70001
    x = random_input((rows, cols), dt, 2.0, seed=cols + 7)
    rng = np.random.default_rng(cols)
    g = (1.0 + 0.25 * rng.standard_normal(cols)).astype(np.float32)
    b = (0.5 * rng.standard_normal(cols)).astype(np.float32)
    if dt == "bf16":
        g, b = wl.f32_to_bf16_bits(g), wl.f32_to_bf16_bits(b)
    xt = to_dev(x)
    full, y = guarded(x.shape, tdtype(dt))
    fk.fk_layernorm_rows(xt, y, to_dev(g), to_dev(b), gelu=True)
    got = to_host(y)
    assert guards_intact(full, x.size)
    assert_ln(got, oracle.layernorm_rows(x, g, b, gelu=True, threads=T), dt, cols,
              g if dt == "f32" else oracle.bf16_to_f32(g),
              b if dt == "f32" else oracle.bf16_to_f32(b), True, f"ln {dt} {rows}x{cols}")
