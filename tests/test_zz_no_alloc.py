"""The allocation-free softmax entry point (fk_softmax_rows_noalloc) against
fk_softmax_rows_ws, through the C ABI, on two calls in a row (the second on
a smaller input), plus its size limit. Needs an MI355X.

The static scratch keeps the previous call's slots: the second, smaller
call must not read them (each slot word carries a per-call tag)."""
import ctypes

import numpy as np
import pytest
import torch

import memory_bound_elementwise_fk_amd as fk
import oracle
from tests.gpu_util import DEV, guarded, guards_intact, random_input, tdtype, to_dev, to_host
from tests.parity import assert_bf16, assert_softmax_f32

pytestmark = pytest.mark.gpu
FK = {"f32": fk.FK_F32, "bf16": fk.FK_BF16}


def noalloc_raw(xt, yt, dt):
    """One call through the C ABI; returns the fk_status."""
    rows, cols = xt.shape
    torch.cuda.synchronize()
    rc = fk.lib().fk_softmax_rows_noalloc(ctypes.c_void_p(xt.data_ptr()),
                                          ctypes.c_void_p(yt.data_ptr()), rows, cols,
                                          xt.stride(0), yt.stride(0), FK[dt], None)
    torch.cuda.synchronize()
    return rc


def reference_ws(x_np, dt):
    xt = to_dev(x_np)
    y = torch.empty_like(xt)
    ws = torch.empty(max(8, fk.fk_softmax_workspace_bytes(*x_np.shape, tdtype(dt))),
                     dtype=torch.uint8, device=DEV)
    fk.fk_softmax_rows_ws(xt, y, ws)
    return to_host(y)


def check(dt, got, ref, what):
    if dt == "f32":
        assert_softmax_f32(got, ref, what)
    else:
        assert_bf16(got, ref, what)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_noalloc_matches_the_workspace_entry_point_on_two_calls(dt):
    # first a large split-path shape, then a smaller one on the same scratch
    shapes = [(1024, 131072), (37, 100003)] if dt == "f32" else [(512, 200001), (9, 70000)]
    for i, shape in enumerate(shapes):
        assert 0 < fk.fk_softmax_workspace_bytes(*shape, tdtype(dt)) <= fk.FK_SOFTMAX_SCRATCH_BYTES
        x = random_input(shape, dt, 3.0, seed=300 + i)
        xt = to_dev(x)
        full, y = guarded(shape, tdtype(dt))
        assert noalloc_raw(xt, y, dt) == fk.FK_OK
        got = to_host(y)
        assert guards_intact(full, x.size), f"call {i}: wrote outside its output"
        want = reference_ws(x, dt)
        bits = np.uint32 if dt == "f32" else np.uint16
        assert np.array_equal(got.view(bits), want.view(bits)), f"call {i}: differs from the ws path"
        if i == 1:  # the smaller call: full oracle comparison too
            check(dt, got, oracle.softmax_rows(x), f"noalloc {dt} {shape}")
        del xt, y, full


def test_noalloc_on_chip_and_in_place_rows():
    x = random_input((64, 1000), "f32", 3.0, seed=311)
    xt = to_dev(x)
    y = torch.empty_like(xt)
    assert noalloc_raw(xt, y, "f32") == fk.FK_OK
    assert_softmax_f32(to_host(y), oracle.softmax_rows(x), "noalloc on chip")
    xw = random_input((3, 70001), "f32", 3.0, seed=312)
    xi = to_dev(xw)
    fk.fk_softmax_rows_noalloc(xi, xi)          # the binding, in place (online path)
    assert_softmax_f32(to_host(xi), oracle.softmax_rows(xw), "noalloc in place")


def test_noalloc_refuses_shapes_beyond_its_scratch():
    # 65537 rows x 2 slices need 2 MiB of slots; refused before any HIP call
    rows, cols = 65537, 40000
    assert fk.fk_softmax_workspace_bytes(rows, cols, torch.float32) > fk.FK_SOFTMAX_SCRATCH_BYTES
    L = fk.lib()
    a, b = 0x7F0000000000, 0x7F8000000000
    assert L.fk_softmax_rows_noalloc(a, b, rows, cols, cols, cols, fk.FK_F32, None) == \
        fk.FK_ERR_UNSUPPORTED
