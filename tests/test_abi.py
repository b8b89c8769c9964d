"""The C ABI of libfusedops on the CPU: symbols and host-side validation.

No compute call is made here: every call below has arguments the library
must reject (or no work at all), and it must do so before any HIP call, so
these run without a GPU.
"""
import ctypes
import re
from pathlib import Path

import pytest

import memory_bound_elementwise_fk_amd as fk

ROOT = Path(__file__).resolve().parents[1]
HEADER = ROOT / "include" / "fusedops.h"

# Plausible, 16-byte aligned fake device addresses: never dereferenced,
# because validation rejects the call first.
A = 0x7F0000000000
B = 0x7F0000100000


@pytest.fixture(scope="module")
def L():
    if not fk.LIB_PATH.exists():
        from memory_bound_elementwise_fk_amd.build import build

        build()
    return fk.lib()


def declared_functions():
    text = HEADER.read_text()
    return sorted(set(re.findall(r"^\s*(?:const\s+char\s*\*|int64_t|int)\s+(fk_\w+)\s*\(",
                                 text, re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for want in ("fk_gelu_tanh", "fk_elementwise_chain", "fk_softmax_rows",
                 "fk_softmax_rows_online", "fk_softmax_rows_ws", "fk_softmax_workspace_bytes",
                 "fk_set_split_wait_limit", "fk_softmax_onchip_max_cols", "fk_copy",
                 "fk_status_string", "fk_layernorm_rows", "fk_layernorm_max_cols",
                 "fk_gelu_tanh_backward", "fk_softmax_rows_backward",
                 "fk_softmax_backward_max_cols", "fk_linear_gelu", "fk_attention_fwd",
                 "fk_softmax_rows_path"):
        assert want in names


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_status_strings(L):
    assert fk.fk_status_string(0) == "ok"
    for st in (-1, -2, -3, -4, 12345):
        assert isinstance(fk.fk_status_string(st), str) and fk.fk_status_string(st)


def test_onchip_capacity_query(L):
    assert L.fk_softmax_onchip_max_cols(fk.FK_F32) == 32768
    assert L.fk_softmax_onchip_max_cols(fk.FK_BF16) == 65536
    assert L.fk_softmax_onchip_max_cols(7) == fk.FK_ERR_INVALID_ARG


@pytest.mark.parametrize("dtype", [fk.FK_F32, fk.FK_BF16])
def test_gelu_validation(L, dtype):
    g = L.fk_gelu_tanh
    assert g(A, B, 0, dtype, None) == fk.FK_OK            # empty: no launch
    assert g(None, None, 0, dtype, None) == fk.FK_OK
    assert g(None, B, 5, dtype, None) == fk.FK_ERR_INVALID_ARG
    assert g(A, None, 5, dtype, None) == fk.FK_ERR_INVALID_ARG
    assert g(A, B, -1, dtype, None) == fk.FK_ERR_INVALID_ARG
    assert g(A, B, 5, 3, None) == fk.FK_ERR_INVALID_ARG
    assert g(A, B, 5, -1, None) == fk.FK_ERR_INVALID_ARG
    assert g(A, A + 4, 5, dtype, None) == fk.FK_ERR_OVERLAP   # partial overlap
    assert g(A + 8, A, 5, dtype, None) == fk.FK_ERR_OVERLAP
    assert g(A, B, 2**62, dtype, None) == fk.FK_ERR_UNSUPPORTED


def _ops(*pairs):
    arr = (fk.fk_op * max(1, len(pairs)))()
    for i, (k, s) in enumerate(pairs):
        arr[i].kind, arr[i].scalar = k, s
    return arr


def test_chain_validation(L):
    c = L.fk_elementwise_chain
    good = _ops((1, 1.0), (3, 0.0), (2, 0.5))
    assert c(A, B, 0, 0, good, 3, None) == fk.FK_OK
    assert c(A, B, 10, 0, None, 3, None) == fk.FK_ERR_INVALID_ARG
    assert c(A, B, 10, 0, good, 0, None) == fk.FK_ERR_INVALID_ARG
    assert c(A, B, 10, 0, _ops(*[(1, 0.0)] * 9), 9, None) == fk.FK_ERR_INVALID_ARG
    assert c(A, B, 10, 0, _ops((5, 1.0)), 1, None) == fk.FK_ERR_INVALID_ARG
    assert c(A, B, 0, 0, _ops((fk.FK_OP_RELU, 0.0)), 1, None) == fk.FK_OK     # ReLU is a kind
    assert c(A, B, 10, 0, _ops((0, 1.0)), 1, None) == fk.FK_ERR_INVALID_ARG
    assert c(A, B, 10, 5, good, 3, None) == fk.FK_ERR_INVALID_ARG
    assert c(None, B, 10, 0, good, 3, None) == fk.FK_ERR_INVALID_ARG
    assert c(A, A + 16, 10, 0, good, 3, None) == fk.FK_ERR_OVERLAP
    # op list validated even when there is no work
    assert c(A, B, 0, 0, _ops((9, 1.0)), 1, None) == fk.FK_ERR_INVALID_ARG


@pytest.mark.parametrize("name", ["fk_softmax_rows", "fk_softmax_rows_online"])
def test_softmax_validation(L, name):
    s = getattr(L, name)
    assert s(A, B, 0, 10, 10, 10, 0, None) == fk.FK_OK       # no rows
    assert s(A, B, 10, 0, 10, 10, 0, None) == fk.FK_OK       # no columns
    assert s(None, None, 0, 0, 0, 0, 0, None) == fk.FK_OK
    assert s(A, B, -1, 10, 10, 10, 0, None) == fk.FK_ERR_INVALID_ARG
    assert s(A, B, 10, -1, 10, 10, 0, None) == fk.FK_ERR_INVALID_ARG
    assert s(A, B, 4, 10, 9, 10, 0, None) == fk.FK_ERR_INVALID_ARG   # ldx < cols
    assert s(A, B, 4, 10, 10, 9, 0, None) == fk.FK_ERR_INVALID_ARG   # ldy < cols
    assert s(None, B, 4, 10, 10, 10, 0, None) == fk.FK_ERR_INVALID_ARG
    assert s(A, None, 4, 10, 10, 10, 0, None) == fk.FK_ERR_INVALID_ARG
    assert s(A, B, 4, 10, 10, 10, 3, None) == fk.FK_ERR_INVALID_ARG  # dtype
    assert s(A, B, 4, 10, 10, 10, 3, None) == fk.FK_ERR_INVALID_ARG
    # in place needs equal strides; any other overlap is rejected
    assert s(A, A, 4, 10, 10, 12, 0, None) == fk.FK_ERR_OVERLAP
    assert s(A, A + 40, 4, 10, 20, 20, 0, None) == fk.FK_ERR_OVERLAP
    assert s(A, B, 2**40, 2**30, 2**30, 2**30, 0, None) == fk.FK_ERR_UNSUPPORTED


def test_softmax_workspace_query(L):
    q = L.fk_softmax_workspace_bytes
    # rows that fit on chip need none
    assert q(32768, 4096, fk.FK_BF16) == 0
    assert q(4096, 32768, fk.FK_F32) == 0
    assert q(10, 65536, fk.FK_BF16) == 0
    assert q(0, 10**6, fk.FK_F32) == 0 and q(10, 0, fk.FK_F32) == 0
    # rows * slices * 16 (two tagged 8-byte words per slice), slices = ceil(cols / 8192)
    assert q(1024, 131072, fk.FK_F32) == 1024 * 16 * 16
    assert q(3, 32769, fk.FK_F32) == 3 * 5 * 16
    assert q(7, 65537, fk.FK_BF16) == 7 * 9 * 16
    assert q(1, 64 * 8192, fk.FK_F32) == 64 * 16
    assert q(1, 64 * 8192 + 1, fk.FK_F32) == 0      # beyond 64 slices: online path
    assert q(-1, 10, fk.FK_F32) == fk.FK_ERR_INVALID_ARG
    assert q(1, 10, 9) == fk.FK_ERR_INVALID_ARG


def test_softmax_ws_validation(L):
    s = L.fk_softmax_rows_ws
    rows, cols = 4, 40000                      # needs a workspace (fp32, 5 slices)
    need = L.fk_softmax_workspace_bytes(rows, cols, fk.FK_F32)
    W = 0x7F0000800000
    assert need > 0
    assert s(A, B, rows, cols, cols, cols, 0, None, 0, None) == fk.FK_ERR_INVALID_ARG
    assert s(A, B, rows, cols, cols, cols, 0, W, need - 8, None) == fk.FK_ERR_INVALID_ARG
    assert s(A, B, rows, cols, cols, cols, 0, W + 4, need, None) == fk.FK_ERR_INVALID_ARG
    assert s(A, B, rows, cols, cols, cols, 0, W, -1, None) == fk.FK_ERR_INVALID_ARG
    assert s(A, B, rows, cols, cols, cols, 0, A + 64, need, None) == fk.FK_ERR_OVERLAP
    assert s(A, B, rows, cols, cols, cols, 0, B, need, None) == fk.FK_ERR_OVERLAP
    assert s(A, B, 0, cols, cols, cols, 0, None, 0, None) == fk.FK_OK     # empty
    assert s(A, B, rows, cols, cols - 1, cols, 0, W, need, None) == fk.FK_ERR_INVALID_ARG


def test_softmax_path_query(L):
    p = L.fk_softmax_rows_path
    A, B = 0x7F0000000000, 0x7F8000000000   # 512 GiB apart: the shapes below never overlap
    F32, BF16 = fk.FK_F32, fk.FK_BF16
    need = L.fk_softmax_workspace_bytes(1024, 131072, F32)
    # rows on chip, whatever the workspace
    assert p(A, B, 4096, 1000, 1000, 1000, F32, 0) == fk.FK_PATH_ONCHIP
    assert p(A, B, 32768, 4096, 4096, 4096, BF16, 0) == fk.FK_PATH_ONCHIP
    assert p(A, B, 3, 32768, 32768, 32768, F32, 0) == fk.FK_PATH_ONCHIP
    assert p(A, B, 3, 65536, 65536, 65536, BF16, 1 << 20) == fk.FK_PATH_ONCHIP
    # wide rows: split with a large enough workspace, online without one
    assert p(A, B, 1024, 131072, 131072, 131072, F32, need) == fk.FK_PATH_SPLIT
    assert p(A, B, 1024, 131072, 131072, 131072, F32, need - 1) == fk.FK_PATH_ONLINE
    assert p(A, B, 1024, 131072, 131072, 131072, F32, 0) == fk.FK_PATH_ONLINE
    assert p(A, B, 3, 32769, 32769, 32769, F32, 3 * 5 * 16) == fk.FK_PATH_SPLIT
    # in place: never split (its fallback would re-read overwritten values)
    assert p(A, A, 1024, 131072, 131072, 131072, F32, need) == fk.FK_PATH_ONLINE
    # more than 64 slices: online
    wide = 64 * 8192 + 1
    assert p(A, B, 2, wide, wide, wide, F32, 1 << 30) == fk.FK_PATH_ONLINE
    # empty work, and arguments the call would refuse
    assert p(A, B, 0, 10, 10, 10, F32, 0) == fk.FK_PATH_NONE
    assert p(None, None, 5, 0, 0, 0, F32, 0) == fk.FK_PATH_NONE
    assert p(A, B, 4, 10, 9, 10, F32, 0) == fk.FK_ERR_INVALID_ARG
    assert p(A, B, 4, 10, 10, 10, F32, -1) == fk.FK_ERR_INVALID_ARG
    assert p(A, A + 40, 4, 10, 20, 20, F32, 0) == fk.FK_ERR_OVERLAP
    assert p(A, B, 4, 10, 10, 10, 9, 0) == fk.FK_ERR_INVALID_ARG
    assert p(A, B, 4, 10, 10, 10, fk.FK_F16, 0) == fk.FK_ERR_UNSUPPORTED


def test_softmax_ws_in_place_ignores_the_workspace(L):
    # wide rows in place take the online path, so the workspace is not
    # validated (it may be NULL); refusals of the row arguments still apply
    s = L.fk_softmax_rows_ws
    assert s(A, A, 4, 40000, 40000, 40001, 0, None, 0, None) == fk.FK_ERR_OVERLAP


def test_split_wait_limit(L):
    prev = L.fk_set_split_wait_limit(123)
    try:
        assert prev >= 0
        assert L.fk_set_split_wait_limit(-1) == fk.FK_ERR_INVALID_ARG
        assert L.fk_set_split_wait_limit(456) == 123
    finally:
        L.fk_set_split_wait_limit(prev)


def test_layernorm_validation(L):
    ln = L.fk_layernorm_rows
    G = 0x7F0000900000
    assert L.fk_layernorm_max_cols(fk.FK_F32) == 32768
    assert L.fk_layernorm_max_cols(fk.FK_BF16) == 65536
    assert L.fk_layernorm_max_cols(5) == fk.FK_ERR_INVALID_ARG
    assert ln(A, B, 0, 10, 10, 10, None, None, 1e-5, 0, 0, None) == fk.FK_OK
    assert ln(A, B, 4, 10, 10, 10, None, None, -1.0, 0, 0, None) == fk.FK_ERR_INVALID_ARG
    assert ln(A, B, 4, 10, 10, 10, None, None, float("nan"), 0, 0, None) == fk.FK_ERR_INVALID_ARG
    assert ln(A, B, 4, 10, 10, 10, None, None, float("inf"), 0, 0, None) == fk.FK_ERR_INVALID_ARG
    assert ln(A, B, 4, 10, 10, 10, None, None, 1e-5, 2, 0, None) == fk.FK_ERR_INVALID_ARG
    assert ln(A, B, 4, 10, 10, 10, None, None, 1e-5, 0, 7, None) == fk.FK_ERR_INVALID_ARG
    assert ln(A, B, 4, 10, 9, 10, None, None, 1e-5, 0, 0, None) == fk.FK_ERR_INVALID_ARG
    assert ln(A, B, 2, 32769, 32769, 32769, None, None, 1e-5, 0, 0, None) == fk.FK_ERR_UNSUPPORTED
    assert ln(A, B, 2, 65537, 65537, 65537, None, None, 1e-5, 0, 1, None) == fk.FK_ERR_UNSUPPORTED
    # gamma / beta must not overlap the output
    assert ln(A, B, 4, 10, 10, 10, B + 8, None, 1e-5, 0, 0, None) == fk.FK_ERR_OVERLAP
    assert ln(A, B, 4, 10, 10, 10, G, B + 100, 1e-5, 0, 0, None) == fk.FK_ERR_OVERLAP
    assert ln(A, A + 8, 4, 10, 10, 10, None, None, 1e-5, 0, 0, None) == fk.FK_ERR_OVERLAP


def test_backward_validation(L):
    gb = L.fk_gelu_tanh_backward
    C = 0x7F0000A00000
    assert gb(A, B, C, 0, 0, None) == fk.FK_OK
    assert gb(None, B, C, 5, 0, None) == fk.FK_ERR_INVALID_ARG
    assert gb(A, None, C, 5, 0, None) == fk.FK_ERR_INVALID_ARG
    assert gb(A, B, None, 5, 0, None) == fk.FK_ERR_INVALID_ARG
    assert gb(A, B, C, -5, 0, None) == fk.FK_ERR_INVALID_ARG
    assert gb(A, B, C, 5, 4, None) == fk.FK_ERR_INVALID_ARG
    assert gb(A, B, A + 4, 5, 0, None) == fk.FK_ERR_OVERLAP       # dx partly over x
    assert gb(A, B, B + 8, 5, 0, None) == fk.FK_ERR_OVERLAP       # dx partly over dy
    sb = L.fk_softmax_rows_backward
    assert L.fk_softmax_backward_max_cols(fk.FK_F32) == 16384
    assert L.fk_softmax_backward_max_cols(fk.FK_BF16) == 32768
    assert L.fk_softmax_backward_max_cols(3) == fk.FK_ERR_INVALID_ARG
    assert sb(A, B, C, 0, 10, 10, 10, 10, 0, None) == fk.FK_OK
    assert sb(A, B, C, 4, 10, 9, 10, 10, 0, None) == fk.FK_ERR_INVALID_ARG
    assert sb(A, B, C, 4, 10, 10, 9, 10, 0, None) == fk.FK_ERR_INVALID_ARG
    assert sb(A, B, C, 4, 10, 10, 10, 9, 0, None) == fk.FK_ERR_INVALID_ARG
    assert sb(A, None, C, 4, 10, 10, 10, 10, 0, None) == fk.FK_ERR_INVALID_ARG
    assert sb(A, B, A + 40, 4, 10, 10, 10, 10, 0, None) == fk.FK_ERR_OVERLAP
    assert sb(A, B, B, 4, 10, 10, 12, 10, 0, None) == fk.FK_ERR_OVERLAP   # in place, other stride
    assert sb(A, B, C, 2, 16385, 16385, 16385, 16385, 0, None) == fk.FK_ERR_UNSUPPORTED
    assert sb(A, B, C, 2, 32769, 32769, 32769, 32769, 1, None) == fk.FK_ERR_UNSUPPORTED


def test_linear_validation(L):
    f = L.fk_linear_gelu
    Y = 0x7F0000B00000
    bf = fk.FK_BF16
    assert f(A, B, None, Y, 0, 10, 16, 16, 16, 10, 1, bf, None) == fk.FK_OK      # M == 0
    assert f(A, B, None, Y, 4, 0, 16, 16, 16, 10, 1, bf, None) == fk.FK_OK      # N == 0
    assert f(A, B, None, Y, -1, 10, 16, 16, 16, 10, 1, bf, None) == fk.FK_ERR_INVALID_ARG
    assert f(A, B, None, Y, 4, 10, 16, 16, 16, 10, 3, bf, None) == fk.FK_ERR_INVALID_ARG  # act
    assert f(A, B, None, Y, 0, 10, 16, 16, 16, 10, fk.FK_ACT_RELU, bf, None) == fk.FK_OK
    assert f(A, B, None, Y, 4, 10, 16, 16, 16, 10, 1, 9, None) == fk.FK_ERR_INVALID_ARG
    assert f(A, B, None, None, 4, 10, 16, 16, 16, 10, 1, bf, None) == fk.FK_ERR_INVALID_ARG
    assert f(None, B, None, Y, 4, 10, 16, 16, 16, 10, 1, bf, None) == fk.FK_ERR_INVALID_ARG
    assert f(A, B, None, Y, 4, 10, 16, 8, 16, 10, 1, bf, None) == fk.FK_ERR_INVALID_ARG  # ldx < K
    assert f(A, B, None, Y, 4, 10, 16, 16, 16, 9, 1, bf, None) == fk.FK_ERR_INVALID_ARG  # ldy < N
    assert f(A, B, None, Y, 4, 10, 16, 16, 16, 10, 1, fk.FK_F32, None) == fk.FK_ERR_UNSUPPORTED
    assert f(A, B, None, Y, 4, 10, 12, 16, 16, 10, 1, bf, None) == fk.FK_ERR_UNSUPPORTED  # K % 8
    assert f(A, B, None, Y, 4, 10, 16, 20, 16, 10, 1, bf, None) == fk.FK_ERR_UNSUPPORTED  # ldx % 8
    assert f(A + 2, B, None, Y, 4, 10, 16, 16, 16, 10, 1, bf, None) == fk.FK_ERR_UNSUPPORTED
    assert f(A, B, None, A + 32, 4, 10, 16, 16, 16, 10, 1, bf, None) == fk.FK_ERR_OVERLAP
    assert f(A, B, Y + 4, Y, 4, 10, 16, 16, 16, 10, 1, bf, None) == fk.FK_ERR_OVERLAP
    # K steps of 32 are counted in 32 bits: K >= 2^36 is refused before any HIP call
    big = 1 << 36
    assert f(A, B, None, Y, 1, 1, big, big, big, 1, 1, bf, None) == fk.FK_ERR_UNSUPPORTED


def test_attention_validation(L):
    import ctypes
    f = L.fk_attention_fwd
    C, D = 0x7F0000C00000, 0x7F0000E00000
    bf = fk.FK_BF16

    def st(*vals):
        return (ctypes.c_int64 * 12)(*vals)

    good = st(*([2 * 3 * 128, 3 * 128, 128] * 4))      # [B=2, H=... ] contiguous, d = 128
    assert f(A, B, C, D, 0, 3, 16, 128, good, 1, bf, None) == fk.FK_OK
    assert f(A, B, C, D, 2, 3, 16, 128, None, 1, bf, None) == fk.FK_ERR_INVALID_ARG
    assert f(A, B, C, D, -1, 3, 16, 128, good, 1, bf, None) == fk.FK_ERR_INVALID_ARG
    assert f(A, B, C, D, 2, 3, 16, 128, good, 2, bf, None) == fk.FK_ERR_INVALID_ARG
    assert f(None, B, C, D, 2, 3, 16, 128, good, 1, bf, None) == fk.FK_ERR_INVALID_ARG
    assert f(A, B, C, D, 2, 3, 16, 64, good, 1, bf, None) == fk.FK_ERR_UNSUPPORTED   # d != 128
    assert f(A, B, C, D, 2, 3, 16, 128, good, 1, fk.FK_F32, None) == fk.FK_ERR_UNSUPPORTED
    assert f(A + 8, B, C, D, 2, 3, 16, 128, good, 1, bf, None) == fk.FK_ERR_UNSUPPORTED
    short = st(*([2 * 3 * 128, 3 * 128, 100] * 4))     # row stride < d
    assert f(A, B, C, D, 2, 3, 16, 128, short, 1, bf, None) == fk.FK_ERR_INVALID_ARG
    odd = st(*([2 * 3 * 136, 3 * 136, 132] * 4))       # stride not a multiple of 8
    assert f(A, B, C, D, 2, 3, 16, 128, odd, 1, bf, None) == fk.FK_ERR_UNSUPPORTED
    assert f(A, B, C, A + 256, 2, 3, 16, 128, good, 1, bf, None) == fk.FK_ERR_OVERLAP
    # more than 2^23 workgroups (B * H * ceil(T / 128))
    assert f(A, B, C, D, 3000, 3000, 16, 128, good, 1, bf, None) == fk.FK_ERR_UNSUPPORTED
    assert f(A, B, C, D, 64, 1024, 128 * 129, 128, good, 1, bf, None) == fk.FK_ERR_UNSUPPORTED
    assert f(A, B, C, D, 1, 1, 1 << 31, 128, good, 1, bf, None) == fk.FK_ERR_UNSUPPORTED


def test_fp16_is_for_linear_and_attention_only(L):
    import ctypes
    f16 = fk.FK_F16
    C, D = 0x7F0000C00000, 0x7F0000E00000
    U = fk.FK_ERR_UNSUPPORTED
    assert L.fk_gelu_tanh(A, B, 5, f16, None) == U
    assert L.fk_elementwise_chain(A, B, 10, f16, _ops((1, 1.0)), 1, None) == U
    for name in ("fk_softmax_rows", "fk_softmax_rows_online"):
        assert getattr(L, name)(A, B, 4, 10, 10, 10, f16, None) == U
    assert L.fk_softmax_rows_ws(A, B, 4, 10, 10, 10, f16, C, 64, None) == U
    assert L.fk_softmax_workspace_bytes(4, 10, f16) == U
    assert L.fk_softmax_onchip_max_cols(f16) == U
    assert L.fk_layernorm_rows(A, B, 4, 10, 10, 10, None, None, 1e-5, 0, f16, None) == U
    assert L.fk_layernorm_max_cols(f16) == U
    assert L.fk_gelu_tanh_backward(A, B, C, 5, f16, None) == U
    assert L.fk_softmax_rows_backward(A, B, C, 4, 10, 10, 10, 10, f16, None) == U
    assert L.fk_softmax_backward_max_cols(f16) == U
    # Linear and attention take it: the same validation as bf16
    li = L.fk_linear_gelu
    assert li(A, B, None, C, 0, 10, 16, 16, 16, 10, 1, f16, None) == fk.FK_OK
    assert li(A, B, None, C, 4, 10, 12, 16, 16, 10, 1, f16, None) == U          # K % 8
    assert li(A, B, None, A + 32, 4, 10, 16, 16, 16, 10, 1, f16, None) == fk.FK_ERR_OVERLAP
    st = (ctypes.c_int64 * 12)(*([2 * 3 * 128, 3 * 128, 128] * 4))
    a = L.fk_attention_fwd
    assert a(A, B, C, D, 0, 3, 16, 128, st, 1, f16, None) == fk.FK_OK
    assert a(A, B, C, D, 2, 3, 16, 64, st, 1, f16, None) == U            # d != 128
    assert a(A, B, C, A + 256, 2, 3, 16, 128, st, 1, f16, None) == fk.FK_ERR_OVERLAP
    assert a(A, B, C, D, 2, 3, 16, 128, st, 1, 3, None) == fk.FK_ERR_INVALID_ARG


def test_copy_validation(L):
    assert L.fk_copy(A, B, 0, None) == fk.FK_OK
    assert L.fk_copy(A, B, -3, None) == fk.FK_ERR_INVALID_ARG
    assert L.fk_copy(None, B, 3, None) == fk.FK_ERR_INVALID_ARG
    assert L.fk_copy(A, A + 1, 3, None) == fk.FK_ERR_OVERLAP


def test_binding_refuses_host_tensors(L):
    torch = pytest.importorskip("torch")
    x = torch.zeros(8)
    with pytest.raises(ValueError):
        fk.fk_gelu_tanh(x, torch.zeros(8))
    with pytest.raises(ValueError):
        fk.fk_softmax_rows(x.view(2, 4), torch.zeros(2, 4))


def test_binding_raises_when_library_missing(monkeypatch, tmp_path):
    monkeypatch.setattr(fk, "_lib", None)
    monkeypatch.setattr(fk, "LIB_PATH", tmp_path / "missing.so")
    with pytest.raises(RuntimeError):
        fk.lib()


def test_product_code_never_imports_the_oracle():
    pkg = ROOT / "memory_bound_elementwise_fk_amd"
    for p in list(pkg.rglob("*.py")) + list(pkg.rglob("*.hip")) + list(pkg.rglob("*.hpp")):
        text = p.read_text()
        assert not re.search(r"^\s*(from|import)\s+oracle\b", text, re.M), p
        assert "liboracle" not in text, p
        assert "oracle.cpp" not in text, p
