"""GPU parity of the split row softmax (rows wider than one workgroup's
registers, sliced over several workgroups that exchange partial max/sum
pairs through a workspace) against the CPU oracle. Needs an MI355X."""
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


def check(dt, got, ref, what):
    if dt == "f32":
        assert_softmax_f32(got, ref, what)
    else:
        assert_bf16(got, ref, what)


def workspace(rows, cols, dt):
    n = fk.fk_softmax_workspace_bytes(rows, cols, tdtype(dt))
    return None if n == 0 else torch.zeros(n, dtype=torch.uint8, device=DEV)


def run_ws(x_np, dt, ws=None):
    rows, cols = x_np.shape
    ws = workspace(rows, cols, dt) if ws is None else ws
    xt = to_dev(x_np)
    full, y = guarded(x_np.shape, tdtype(dt))
    fk.fk_softmax_rows_ws(xt, y, ws)
    got = to_host(y)
    assert guards_intact(full, x_np.size), "softmax wrote outside its output"
    if ws is not None:
        assert int(ws.count_nonzero()) == 0, "workspace not left zeroed"
    return got


def run_self(x_np, dt):
    xt = to_dev(x_np)
    full, y = guarded(x_np.shape, tdtype(dt))
    fk.fk_softmax_rows(xt, y)
    got = to_host(y)
    assert guards_intact(full, x_np.size)
    return got


# slices are 8192 columns; on-chip capacity is 32768 fp32 / 65536 bf16 columns
WIDTHS = {"f32": [32769, 40000, 65536, 100003, 131072, 64 * 8192],
          "bf16": [65537, 100003, 131072, 262147, 64 * 8192]}


@pytest.mark.parametrize("dt,cols", [(d, c) for d, cs in WIDTHS.items() for c in cs])
def test_split_widths(dt, cols):
    assert fk.fk_softmax_workspace_bytes(3, cols, tdtype(dt)) > 0   # the split path applies
    x = random_input((3, cols), dt, 3.0, seed=cols + 1)
    ref = oracle.softmax_rows(x)
    check(dt, run_ws(x, dt), ref, f"split ws {dt} cols={cols}")
    check(dt, run_self(x, dt), ref, f"split self-managed {dt} cols={cols}")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_beyond_64_slices_falls_back_to_online(dt):
    cols = 64 * 8192 + 5
    assert fk.fk_softmax_workspace_bytes(2, cols, tdtype(dt)) == 0
    x = random_input((2, cols), dt, 3.0, seed=77)
    check(dt, run_self(x, dt), oracle.softmax_rows(x), "online beyond 64 slices")


def test_c5a_full_size_split_and_online():
    x = wl.make_input("C5a")
    ref = oracle.softmax_rows(x, threads=T)
    xt = to_dev(x)
    y = torch.empty_like(xt)
    ws = workspace(*x.shape, "f32")
    fk.fk_softmax_rows_ws(xt, y, ws)
    got = to_host(y)
    assert_softmax_f32(got, ref, "C5a split")
    assert np.max(np.abs(got.astype(np.float64).sum(axis=1) - 1.0)) < 1e-5
    assert int(ws.count_nonzero()) == 0
    fk.fk_softmax_rows_online(xt, y)
    assert_softmax_f32(to_host(y), ref, "C5a online")
    del xt, y


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_forced_fallback_statistics(dt):
    # a zero wait bound sends every block onto the streamed row statistics
    cols = 3 * 8192 + 70000 if dt == "f32" else 70001
    x = random_input((5, cols), dt, 4.0, seed=21)
    ref = oracle.softmax_rows(x)
    prev = fk.fk_set_split_wait_limit(0)
    try:
        got = run_ws(x, dt)
    finally:
        fk.fk_set_split_wait_limit(prev)
    check(dt, got, ref, f"forced fallback {dt}")


def test_split_rows_are_bitwise_reproducible_and_slices_agree():
    x = random_input((8, 131072), "f32", 3.0, seed=31)
    a = run_ws(x, "f32")
    b = run_ws(x, "f32")
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    # a constant row: every slice must normalise with the same (M, L)
    c = np.full((2, 40960), 1.5, np.float32)
    got = run_ws(c, "f32")
    assert np.all(got == got[0, 0])


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_split_strided_unaligned_in_place(dt):
    rows, cols, ld = 3, 70001, 70016
    xbig = random_input((rows, ld), dt, 3.0, seed=41)
    ref = oracle.softmax_rows(np.ascontiguousarray(xbig[:, :cols]))
    # strided rows keep their padding
    xt = to_dev(xbig)[:, :cols]
    full, ybig = guarded((rows, ld), tdtype(dt))
    fk.fk_softmax_rows_ws(xt, ybig[:, :cols], workspace(rows, cols, dt))
    got = to_host(ybig)
    assert guards_intact(full, rows * ld)
    check(dt, got[:, :cols], ref, "split strided")
    assert np.all(got[:, cols:].view(np.uint16 if dt == "bf16" else np.uint32) == CANARY_BITS[dt])
    # unaligned base (scalar path)
    flat = random_input((rows * cols + 1,), dt, 3.0, seed=42)
    xu = to_dev(flat)[1:].view(rows, cols)
    yu = torch.empty(rows * cols + 1, dtype=tdtype(dt), device=DEV)[1:].view(rows, cols)
    fk.fk_softmax_rows_ws(xu, yu, workspace(rows, cols, dt))
    check(dt, to_host(yu), oracle.softmax_rows(flat[1:].reshape(rows, cols)), "split unaligned")
    # in place
    xi = to_dev(np.ascontiguousarray(xbig[:, :cols]))
    fk.fk_softmax_rows_ws(xi, xi, workspace(rows, cols, dt))
    check(dt, to_host(xi), ref, "split in place")


def test_split_special_rows():
    cols = 40000
    x = random_input((5, cols), "f32", 2.0, seed=51)
    x[0, 30000] = np.nan                 # NaN in the last slice -> whole row NaN
    x[1, :] = -np.inf                    # all -inf -> NaN
    x[2, 100] = np.inf                   # +inf -> NaN
    x[3, :8192] = -np.inf                # one slice entirely -inf: it contributes nothing
    x[4, 12345] = 200.0                  # one dominant entry in a middle slice
    got = run_ws(x, "f32")
    ref = oracle.softmax_rows(x)
    assert_softmax_f32(got, ref, "split specials")
    assert np.all(np.isnan(got[0:3]))
    assert np.all(got[3, :8192] == 0)
    assert got[4, 12345] == np.float32(1.0) or abs(got[4, 12345] - 1.0) < 2e-6


def test_split_many_rows_workspace_reuse():
    # many rows through one workspace, twice, including a smaller second call
    ws = workspace(600, 66000, "bf16")
    assert ws is not None
    x2 = random_input((600, 66000), "bf16", 8.0, seed=62)
    check("bf16", run_ws(x2, "bf16", ws), oracle.softmax_rows(x2, threads=T), "first call")
    x3 = random_input((17, 90000), "bf16", 8.0, seed=63)
    check("bf16", run_ws(x3, "bf16", ws), oracle.softmax_rows(x3), "second call")
