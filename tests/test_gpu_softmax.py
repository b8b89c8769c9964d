"""GPU parity of the row-softmax kernels against the CPU oracle (needs MI355X)."""
import numpy as np
import pytest
import torch

import memory_bound_elementwise_fk_amd as fk
import oracle
from memory_bound_elementwise_fk_amd import workloads as wl
from tests.gpu_util import CANARY_BITS, DEV, guarded, guards_intact, random_input, tdtype, \
    to_dev, to_host
from tests.parity import assert_bf16, assert_softmax_f32

pytestmark = pytest.mark.gpu
T = oracle.default_threads()

PATHS = {"single": fk.fk_softmax_rows, "online": fk.fk_softmax_rows_online}


def check(dt, got, ref, what):
    if dt == "f32":
        assert_softmax_f32(got, ref, what)
    else:
        assert_bf16(got, ref, what)


def run(x_np, dt, path="single"):
    xt = to_dev(x_np)
    full, y = guarded(x_np.shape, tdtype(dt))
    PATHS[path](xt, y)
    got = to_host(y)
    assert guards_intact(full, x_np.size), "softmax wrote outside its output"
    return got


# ------------------------------------------------------- full workloads ---
def test_c2_softmax_fp32_full_size():
    x = wl.make_input("C2")
    got = run(x, "f32")
    assert_softmax_f32(got, oracle.softmax_rows(x, threads=T), "C2")
    assert np.max(np.abs(got.astype(np.float64).sum(axis=1) - 1.0)) < 1e-5


def test_c4_softmax_bf16_full_size():
    x = wl.make_input("C4")
    xt = to_dev(x)
    y = torch.empty_like(xt)
    fk.fk_softmax_rows(xt, y)
    got = to_host(y)
    del xt, y
    assert_bf16(got, oracle.softmax_rows(x, threads=T), "C4")
    assert np.all(got[x == wl.BF16_MINUS_1E4] == 0)        # masked entries are exactly 0


def test_c5a_softmax_fp32_full_size_no_workspace():
    # wider than on-chip capacity: without a workspace fk_softmax_rows takes
    # the online path (it allocates nothing)
    x = wl.make_input("C5a")
    assert x.shape[1] > fk.fk_softmax_onchip_max_cols(torch.float32)
    assert fk.fk_softmax_workspace_bytes(*x.shape, torch.float32) > 0
    xt = to_dev(x)
    y = torch.empty_like(xt)
    assert fk.fk_softmax_rows_path(xt, y) == fk.FK_PATH_ONLINE
    fk.fk_softmax_rows(xt, y)
    got = to_host(y)
    del xt, y
    assert_softmax_f32(got, oracle.softmax_rows(x, threads=T), "C5a")
    assert np.max(np.abs(got.astype(np.float64).sum(axis=1) - 1.0)) < 1e-5


# ------------------------------------------------------------- shapes -----
# ragged widths; widths that fill a single-pass row shape exactly (256 * 2^k,
# and 1536 ... 24576 for the 3-, 5-, 6- and 12-wave shapes: the unmasked
# kernel variant) for both dtypes; multiples of the vector inside a shape
# (1000, 3000, 5000, 12000: the per-vector masks)
COLS = [1, 2, 3, 5, 63, 64, 65, 255, 256, 257, 512, 1000, 1023, 1024, 1025, 1536, 2047, 2048, 2049,
        2560, 3000, 3072, 4095, 4096, 4097, 5000, 5120, 6144, 8192, 8193, 10240, 12000, 12288,
        16384, 16385, 24576, 32768, 32769, 65536, 65537, 100_003]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("cols", COLS)
def test_softmax_widths_both_paths(dt, cols):
    rows = 3 if cols > 8192 else 17
    x = random_input((rows, cols), dt, 3.0, seed=cols)
    ref = oracle.softmax_rows(x)
    for path in ("single", "online"):
        check(dt, run(x, dt, path), ref, f"{dt} cols={cols} {path}")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_softmax_single_row_and_many_rows(dt):
    x1 = random_input((1, 777), dt, 2.0, seed=1)
    check(dt, run(x1, dt), oracle.softmax_rows(x1), "one row")
    xm = random_input((40_001, 33), dt, 2.0, seed=2)
    check(dt, run(xm, dt), oracle.softmax_rows(xm, threads=T), "many rows")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("path", ["single", "online"])
@pytest.mark.parametrize("cols,ldx,ldy", [(1000, 1004, 1016), (1000, 1001, 1003), (300, 300, 301)])
def test_softmax_strided_rows_keep_padding(dt, path, cols, ldx, ldy):
    rows = 9
    xbig = random_input((rows, ldx), dt, 3.0, seed=cols + ldx)
    xt = to_dev(xbig)[:, :cols]
    full, ybig = guarded((rows, ldy), tdtype(dt))
    y = ybig[:, :cols]
    PATHS[path](xt, y)
    got = to_host(ybig)
    assert guards_intact(full, rows * ldy)
    check(dt, got[:, :cols], oracle.softmax_rows(np.ascontiguousarray(xbig[:, :cols])),
          f"strided {dt} {path}")
    pad = got[:, cols:].view(np.uint16 if dt == "bf16" else np.uint32)
    assert np.all(pad == CANARY_BITS[dt]), "row padding was written"


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("path", ["single", "online"])
def test_softmax_unaligned_base(dt, path):
    rows, cols = 5, 999
    flat = random_input((rows * cols + 3,), dt, 3.0, seed=7)
    xt = to_dev(flat)[1:1 + rows * cols].view(rows, cols)
    full, ybuf = guarded((rows * cols + 3,), tdtype(dt))
    y = ybuf[2:2 + rows * cols].view(rows, cols)
    PATHS[path](xt, y)
    got = to_host(y)
    assert guards_intact(full, rows * cols + 3)
    check(dt, got, oracle.softmax_rows(flat[1:1 + rows * cols].reshape(rows, cols)),
          f"unaligned {dt} {path}")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("path", ["single", "online"])
def test_softmax_in_place(dt, path):
    x = random_input((64, 1000), dt, 3.0, seed=8)
    xt = to_dev(x)
    PATHS[path](xt, xt)
    check(dt, to_host(xt), oracle.softmax_rows(x), f"in place {dt} {path}")


# ------------------------------------------------------- special rows -----
@pytest.mark.parametrize("path", ["single", "online"])
def test_softmax_special_rows_fp32(path):
    ninf = -np.inf
    x = np.float32([[1.0, np.nan, 2.0, 0.0], [1.0, np.inf, 2.0, 0.0],
                    [ninf, ninf, ninf, ninf], [ninf, 0.0, 1.0, ninf],
                    [5.0, 5.0, 5.0, 5.0], [1e30, -1e30, 0.0, 1e30],
                    [0.0, -100.0, -90.0, -120.0]])
    got = run(x, "f32", path)
    ref = oracle.softmax_rows(x)
    assert_softmax_f32(got, ref, f"special {path}")
    assert np.all(np.isnan(got[0:3]))
    assert got[3][0] == 0 and got[3][3] == 0
    assert np.all(got[4] == np.float32(0.25))
    # a result in the subnormal range is not flushed: e^-90 / (1 + ...) ~ 8.2e-40.
    # Its relative error is set by the fp32 exponent argument (x - m) log2(e)
    # ~ -129.8, rounded to half an ulp (2^-18), i.e. ~2.6e-6 relative in the
    # power, plus the exp2 and final subnormal rounding (~1.7e-6 each here).
    rel = abs(float(got[6][2]) - float(ref[6][2])) / float(ref[6][2])
    assert got[6][2] > 0 and rel <= 1e-5


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("path", ["single", "online"])
def test_softmax_single_column_and_constant_rows(dt, path):
    one = np.ones(1, np.float32)
    x1 = random_input((100, 1), dt, 50.0, seed=3)
    got = run(x1, dt, path)
    ref = oracle.softmax_rows(x1)
    assert np.array_equal(got, ref)
    if dt == "f32":
        assert np.all(got == one)
    # exp of the max element is exactly 1, sums of ones are exact, and 1/2^k
    # is exact, so constant rows of 2^k columns are bit-exact
    for k in (1, 6, 10, 13):
        cols = 1 << k
        xc = np.full((4, cols), 2.5, np.float32)
        xc = xc if dt == "f32" else wl.f32_to_bf16_bits(xc).reshape(4, cols)
        assert np.array_equal(run(xc, dt, path), oracle.softmax_rows(xc)), f"constant {cols}"


@pytest.mark.parametrize("path", ["single", "online"])
def test_softmax_shift_invariance(path):
    rng = np.random.default_rng(5)
    x = (np.round(rng.standard_normal((32, 1000)) * 3 * 1024) / 1024).astype(np.float32)
    xs = x + np.float32(800.0)
    a, b = run(x, "f32", path), run(xs, "f32", path)
    ref = oracle.softmax_rows(x)
    assert_softmax_f32(a, ref, "unshifted")
    assert_softmax_f32(b, ref, "shifted by 800")


def test_online_and_single_pass_agree():
    for dt in ("f32", "bf16"):
        x = random_input((50, 4096), dt, 8.0, seed=12)
        a, b = run(x, dt, "single"), run(x, dt, "online")
        if dt == "f32":
            assert np.max(np.abs(a - b)) <= 2e-6
        else:
            assert_bf16(a, b, "online vs single")


def test_softmax_runs_are_bitwise_reproducible():
    for path in ("single", "online"):
        x = to_dev(random_input((64, 40_000), "f32", 3.0, seed=13))
        y1, y2 = torch.empty_like(x), torch.empty_like(x)
        PATHS[path](x, y1)
        PATHS[path](x, y2)
        assert torch.equal(y1.view(torch.int32), y2.view(torch.int32)), path


@pytest.mark.parametrize("cols", [1, 3])
def test_softmax_rows_beyond_one_launch_grid(cols):
    # 2^25 + 5 rows of 1 or 3 fp32 columns: more workgroups than one launch's
    # 2^31 work-items hold, so the kernel strides over rows; sampled rows
    rows = (1 << 25) + 5
    gen = torch.Generator(device=DEV)
    gen.manual_seed(cols)
    x = torch.randn(rows, cols, dtype=torch.float32, device=DEV, generator=gen).mul_(3)
    y = fk.softmax_rows(x)
    rng = np.random.default_rng(cols)
    idx = np.unique(np.concatenate([rng.integers(0, rows, 200_000), np.arange(rows - 100, rows)]))
    it = torch.from_numpy(idx).to(DEV)
    xs, ys = wl.from_torch(x[it]), wl.from_torch(y[it])
    del x, y
    torch.cuda.empty_cache()
    check("f32", ys, oracle.softmax_rows(xs), f"softmax {rows}x{cols}, sampled rows")
