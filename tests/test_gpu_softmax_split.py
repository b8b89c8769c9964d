"""GPU parity of the split row softmax (rows wider than one workgroup's
registers, sliced over several workgroups that exchange partial max/sum
pairs through a caller workspace) against the CPU oracle, and of the online
path that fk_softmax_rows takes for the same rows without a workspace.
Needs an MI355X."""
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


def workspace(rows, cols, dt, fill=None):
    """A workspace for the split path: uninitialised memory (any contents
    are valid), or filled with the byte `fill`."""
    n = fk.fk_softmax_workspace_bytes(rows, cols, tdtype(dt))
    if n == 0:
        return None
    ws = torch.empty(n, dtype=torch.uint8, device=DEV)
    if fill is not None:
        ws.fill_(fill)
    return ws


def run_ws(x_np, dt, ws=None):
    rows, cols = x_np.shape
    ws = workspace(rows, cols, dt) if ws is None else ws
    xt = to_dev(x_np)
    full, y = guarded(x_np.shape, tdtype(dt))
    if ws is not None:
        assert fk.fk_softmax_rows_path(xt, y, ws.numel()) == fk.FK_PATH_SPLIT
    fk.fk_softmax_rows_ws(xt, y, ws)
    got = to_host(y)
    assert guards_intact(full, x_np.size), "softmax wrote outside its output"
    return got


def run_self(x_np, dt):
    """fk_softmax_rows: no workspace, so wide rows take the online path."""
    xt = to_dev(x_np)
    full, y = guarded(x_np.shape, tdtype(dt))
    assert fk.fk_softmax_rows_path(xt, y) == fk.FK_PATH_ONLINE
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
    check(dt, run_self(x, dt), ref, f"online (no workspace) {dt} cols={cols}")


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
    fk.fk_softmax_rows_online(xt, y)
    assert_softmax_f32(to_host(y), ref, "C5a online")
    fk.fk_softmax_rows(xt, y)
    assert_softmax_f32(to_host(y), ref, "C5a through fk_softmax_rows (online)")
    del xt, y


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_forced_fallback_statistics(dt):
    # a zero wait bound: every block polls once, and those that do not find
    # all of their row's partials already published (all but the last ones
    # to publish) compute the row statistics by streaming the row
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
    check(dt, to_host(xi), ref, "in place (online path)")


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


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("fill", [0x00, 0xFF, "random"])
def test_dirty_workspace_gives_correct_rows(dt, fill):
    # whatever the workspace holds -- zeros, all ones, random bytes -- no
    # slot counts for this call without its tag
    rows, cols = 6, 70001 if dt == "f32" else 140001
    n = fk.fk_softmax_workspace_bytes(rows, cols, tdtype(dt))
    if fill == "random":
        ws = torch.from_numpy(np.random.default_rng(7).integers(0, 256, n, dtype=np.uint8)).to(DEV)
    else:
        ws = workspace(rows, cols, dt, fill)
    x = random_input((rows, cols), dt, 4.0, seed=71)
    check(dt, run_ws(x, dt, ws), oracle.softmax_rows(x), f"dirty workspace {fill}")


@pytest.mark.parametrize("wait", [None, 0])
def test_stale_partials_of_a_previous_call_are_ignored(wait):
    # the first call leaves its own tagged partials in the workspace; a
    # second call on other data with the same shape must not read them,
    # whether its blocks wait for their row's slices or not
    rows, cols = 9, 100003
    ws = workspace(rows, cols, "f32")
    a = random_input((rows, cols), "f32", 3.0, seed=81)
    b = random_input((rows, cols), "f32", 3.0, seed=82)
    b[:, 5] += 30.0  # a different max in every row
    assert_softmax_f32(run_ws(a, "f32", ws), oracle.softmax_rows(a), "first call")
    assert int(ws.count_nonzero()) > 0  # partials left behind, not cleared
    prev = fk.fk_set_split_wait_limit(wait) if wait is not None else None
    try:
        got = run_ws(b, "f32", ws)
    finally:
        if prev is not None:
            fk.fk_set_split_wait_limit(prev)
    assert_softmax_f32(got, oracle.softmax_rows(b), "second call, stale partials present")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_in_place_wide_rows_take_the_online_path(dt):
    # in place, wide rows never take the split path, so no block can re-read
    # values another slice has already overwritten -- with a zero wait
    # bound too (every split block that polls in vain would re-read x)
    rows, cols = 4, 3 * 8192 + 70000 if dt == "f32" else 140003
    x = random_input((rows, cols), dt, 4.0, seed=91)
    ref = oracle.softmax_rows(x)
    xt = to_dev(x)
    ws = workspace(rows, cols, dt)
    assert fk.fk_softmax_rows_path(xt, xt, ws.numel()) == fk.FK_PATH_ONLINE
    prev = fk.fk_set_split_wait_limit(0)
    try:
        fk.fk_softmax_rows_ws(xt, xt, ws)
        got = to_host(xt)
    finally:
        fk.fk_set_split_wait_limit(prev)
    check(dt, got, ref, f"in place {dt}")


def test_split_many_rows_workspace_reuse():
    # many rows through one workspace, twice, including a smaller second call
    ws = workspace(600, 66000, "bf16")
    assert ws is not None
    x2 = random_input((600, 66000), "bf16", 8.0, seed=62)
    check("bf16", run_ws(x2, "bf16", ws), oracle.softmax_rows(x2, threads=T), "first call")
    x3 = random_input((17, 90000), "bf16", 8.0, seed=63)
    check("bf16", run_ws(x3, "bf16", ws), oracle.softmax_rows(x3), "second call")


# The online path for aligned rows keeps whole 8192-column chunks on chip
# (fp32: 12 in registers + 4 in LDS = 131072 columns; bf16: 24 + 8 = 262144)
# and streams the rest twice, a ragged row's partial last chunk always among
# the streamed ones. Widths around every transition: inside the first chunk,
# the register/LDS boundary, all resident, one streamed chunk, ragged ends.
K = 8192
STAGED = {"f32": [1, 1000, K - 1, K, K + 1, 12 * K, 12 * K + 7, 13 * K + 1, 16 * K, 16 * K + 1,
                  17 * K, 18 * K + 4095, 300003],
          "bf16": [3, K, 24 * K, 24 * K + 9, 32 * K, 32 * K + 1, 33 * K, 400001]}


@pytest.mark.parametrize("dt,cols", [(d, c) for d, cs in STAGED.items() for c in cs])
def test_online_staged_chunk_boundaries(dt, cols):
    rows = 3
    x = random_input((rows, cols), dt, 3.0, seed=cols % 1000 + 5)
    if cols > 20000:
        x[1, cols - 1] = x[1].max() + (4.0 if dt == "f32" else 0)   # the max in the last chunk
        x[2, 0] = x[2].max() + (4.0 if dt == "f32" else 0)          # the max in the first
    xt = to_dev(x)
    full, y = guarded(x.shape, tdtype(dt))
    fk.fk_softmax_rows_online(xt, y)
    got = to_host(y)
    assert guards_intact(full, x.size), "online softmax wrote outside its output"
    check(dt, got, oracle.softmax_rows(x), f"online staged {dt} cols={cols}")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_online_staged_strided_in_place_and_many_rows(dt):
    cols, ld = 7 * 16384 + 3, 7 * 16384 + 64
    rows = 300 if dt == "bf16" else 270          # more rows than CUs: several per workgroup slot
    xbig = random_input((rows, ld), dt, 5.0, seed=97)
    xs = np.ascontiguousarray(xbig[:, :cols])
    ref = oracle.softmax_rows(xs, threads=T)
    full, ybig = guarded((rows, ld), tdtype(dt))
    fk.fk_softmax_rows_online(to_dev(xbig)[:, :cols], ybig[:, :cols])
    got = to_host(ybig)
    assert guards_intact(full, rows * ld)
    check(dt, got[:, :cols], ref, "online strided")
    assert np.all(got[:, cols:].view(np.uint16 if dt == "bf16" else np.uint32) == CANARY_BITS[dt])
    xi = to_dev(xs)
    fk.fk_softmax_rows_online(xi, xi)
    check(dt, to_host(xi), ref, "online in place")


# Rows of whole chunks that stay on chip run the rolling kernel: a persistent
# grid (one workgroup per CU) whose pass 2 loads the workgroup's next row
# into each chunk's registers or LDS words as soon as the current row's
# chunk is stored. More rows than CUs (several per workgroup, a ragged last
# round), rows that differ sharply from their neighbours (a NaN row, an all
# -inf row, a row shifted far up), in place too.
@pytest.mark.parametrize("dt,chunks", [("f32", 5), ("f32", 12), ("f32", 16), ("bf16", 3),
                                       ("bf16", 24), ("bf16", 32)])
def test_online_rolling_many_rows(dt, chunks):
    cols = chunks * K
    rows = 701 if chunks * K * 4 <= (1 << 19) else 300
    x = random_input((rows, cols), dt, 3.0, seed=chunks * 11 + len(dt))
    if dt == "f32":
        x[257, 5] = np.nan
        x[300, :] = -np.inf
        x[258] += 200.0
    ref = oracle.softmax_rows(x, threads=T)
    xt = to_dev(x)
    full, y = guarded(x.shape, tdtype(dt))
    fk.fk_softmax_rows_online(xt, y)
    got = to_host(y)
    assert guards_intact(full, x.size), "rolling softmax wrote outside its output"
    check(dt, got, ref, f"rolling {dt} cols={cols} rows={rows}")
    fk.fk_softmax_rows_online(xt, xt)
    check(dt, to_host(xt), ref, f"rolling in place {dt} cols={cols}")


def test_online_staged_special_rows():
    cols = 18 * K + 5
    x = random_input((5, cols), "f32", 2.0, seed=53)
    x[0, cols - 2] = np.nan            # NaN in the streamed partial chunk -> whole row NaN
    x[1, :] = -np.inf                  # all -inf -> NaN
    x[2, 13 * K + 10] = np.inf         # +inf in an LDS chunk -> NaN
    x[3, :16 * K] = -np.inf            # every resident chunk -inf: only streamed values count
    x[4, 6 * K + 1] = 300.0            # one dominant entry in a register chunk
    xt = to_dev(x)
    y = torch.empty_like(xt)
    fk.fk_softmax_rows_online(xt, y)
    got = to_host(y)
    assert_softmax_f32(got, oracle.softmax_rows(x), "online specials")
    assert np.all(np.isnan(got[0:3]))
    assert np.all(got[3, :16 * K] == 0)
    assert abs(float(got[4, 6 * K + 1]) - 1.0) < 2e-6
