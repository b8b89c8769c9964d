"""CPU oracle for the fused memory-bound kernels -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product path (the HIP library and
its Python binding) never imports, links or calls it, and the two share no
code: the oracle is plain C++ in double precision (``oracle.cpp``) built with
g++, plus the pure-Python tiling model in ``tiling.py``.

Arrays are numpy: fp32 as ``float32``, bf16 as ``uint16`` bit patterns.
Every function cites the passage it follows in ``oracle.cpp``.
"""
from __future__ import annotations

import ctypes
import os
from pathlib import Path

import numpy as np

from . import tiling  # noqa: F401  (re-exported)

_HERE = Path(__file__).resolve().parent
LIB_PATH = _HERE / "liboracle.so"

OP_ADD_SCALAR = 1
OP_MUL_SCALAR = 2
OP_GELU_TANH = 3
OP_RELU = 4

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not LIB_PATH.exists():
        from .build_oracle import build

        build()
    lib = ctypes.CDLL(str(LIB_PATH))
    i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    sig = {
        "oracle_f32_to_bf16": ([vp, vp, i64], None),
        "oracle_bf16_to_f32": ([vp, vp, i64], None),
        "oracle_gelu_tanh_f64": ([vp, vp, i64], None),
        "oracle_gelu_tanh_literal_f64": ([vp, vp, i64], None),
        "oracle_gelu_tanh_f32": ([vp, vp, i64, i32], None),
        "oracle_gelu_tanh_bf16": ([vp, vp, i64, i32], None),
        "oracle_chain_f32": ([vp, vp, i64, vp, vp, i32, i32], i32),
        "oracle_chain_bf16": ([vp, vp, i64, vp, vp, i32, i32], i32),
        "oracle_softmax_rows_f64": ([vp, vp, i64, i64, i64, i64], i32),
        "oracle_softmax_rows_f32": ([vp, vp, i64, i64, i64, i64, i32], i32),
        "oracle_softmax_rows_bf16": ([vp, vp, i64, i64, i64, i64, i32], i32),
        "oracle_gelu_tanh_grad_f64": ([vp, vp, i64], None),
        "oracle_gelu_tanh_bwd_f32": ([vp, vp, vp, i64, i32], None),
        "oracle_gelu_tanh_bwd_bf16": ([vp, vp, vp, i64, i32], None),
        "oracle_softmax_bwd_rows_f64": ([vp, vp, vp, i64, i64], i32),
        "oracle_softmax_bwd_rows_f32": ([vp, vp, vp, i64, i64, i32], i32),
        "oracle_softmax_bwd_rows_bf16": ([vp, vp, vp, i64, i64, i32], i32),
        "oracle_layernorm_rows_f64": ([vp, vp, i64, i64, i64, i64, vp, vp, ctypes.c_double, i32],
                                      i32),
        "oracle_layernorm_rows_f32": ([vp, vp, i64, i64, i64, i64, vp, vp, ctypes.c_double, i32,
                                       i32], i32),
        "oracle_layernorm_rows_bf16": ([vp, vp, i64, i64, i64, i64, vp, vp, ctypes.c_double, i32,
                                        i32], i32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def default_threads() -> int:
    """Threads the oracle may use: the process's CPU share, capped by OMP_NUM_THREADS."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    cap = os.environ.get("OMP_NUM_THREADS")
    if cap and cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


# ------------------------------------------------------------ rounding ----
def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even, NaN kept (quiet)."""
    x = _c(x, np.float32)
    y = np.empty(x.shape, np.uint16)
    _load().oracle_f32_to_bf16(_ptr(x), _ptr(y), x.size)
    return y


def bf16_to_f32(x: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 (exact widening)."""
    x = _c(x, np.uint16)
    y = np.empty(x.shape, np.float32)
    _load().oracle_bf16_to_f32(_ptr(x), _ptr(y), x.size)
    return y


# ---------------------------------------------------------------- GELU ----
def gelu_tanh_f64(x: np.ndarray) -> np.ndarray:
    """The real tanh-GELU in double (cancellation-free form), unrounded."""
    x = _c(x, np.float64)
    y = np.empty_like(x)
    _load().oracle_gelu_tanh_f64(_ptr(x), _ptr(y), x.size)
    return y


def gelu_tanh_literal_f64(x: np.ndarray) -> np.ndarray:
    """The literal 0.5 x (1 + tanh u) in double, unrounded (for the pins)."""
    x = _c(x, np.float64)
    y = np.empty_like(x)
    _load().oracle_gelu_tanh_literal_f64(_ptr(x), _ptr(y), x.size)
    return y


def gelu_tanh(x: np.ndarray, threads: int = 1) -> np.ndarray:
    """tanh-GELU of fp32 (float32) or bf16 (uint16) data, same dtype out."""
    lib = _load()
    if x.dtype == np.uint16:
        x = _c(x, np.uint16)
        y = np.empty_like(x)
        lib.oracle_gelu_tanh_bf16(_ptr(x), _ptr(y), x.size, threads)
        return y
    x = _c(x, np.float32)
    y = np.empty_like(x)
    lib.oracle_gelu_tanh_f32(_ptr(x), _ptr(y), x.size, threads)
    return y


# ---------------------------------------------------------------- chain ---
def chain(x: np.ndarray, ops, threads: int = 1) -> np.ndarray:
    """Apply ``ops`` ((kind, scalar) pairs, in order) elementwise, fp32 intermediates."""
    kinds = np.array([k for k, _ in ops], np.int32)
    scal = np.array([s for _, s in ops], np.float32)
    lib = _load()
    if x.dtype == np.uint16:
        x = _c(x, np.uint16)
        y = np.empty_like(x)
        rc = lib.oracle_chain_bf16(_ptr(x), _ptr(y), x.size, _ptr(kinds), _ptr(scal), len(ops),
                                   threads)
    else:
        x = _c(x, np.float32)
        y = np.empty_like(x)
        rc = lib.oracle_chain_f32(_ptr(x), _ptr(y), x.size, _ptr(kinds), _ptr(scal), len(ops),
                                  threads)
    if rc != 0:
        raise ValueError(f"invalid op list {ops!r}")
    return y


# ---------------------------------------------------------------- softmax -
def softmax_rows(x: np.ndarray, threads: int = 1, out: np.ndarray | None = None) -> np.ndarray:
    """Softmax along the last axis of a 2-D array (float64, float32 or bf16 uint16).

    Row strides of ``x`` (and of ``out`` if given) are honoured; entries of
    ``out`` past ``cols`` in each row are left untouched.
    """
    if x.ndim != 2:
        raise ValueError("softmax_rows expects a 2-D array")
    rows, cols = x.shape
    if x.strides[1] != x.itemsize:
        x = np.ascontiguousarray(x)
    if out is None:
        out = np.empty((rows, cols), x.dtype)
    if out.dtype != x.dtype or out.shape != x.shape or out.strides[1] != out.itemsize:
        raise ValueError("out must match x in dtype and shape, unit column stride")
    ldx = x.strides[0] // x.itemsize if rows > 1 else cols
    ldy = out.strides[0] // out.itemsize if rows > 1 else cols
    lib = _load()
    if x.dtype == np.float64:
        rc = lib.oracle_softmax_rows_f64(_ptr(x), _ptr(out), rows, cols, ldx, ldy)
    elif x.dtype == np.float32:
        rc = lib.oracle_softmax_rows_f32(_ptr(x), _ptr(out), rows, cols, ldx, ldy, threads)
    elif x.dtype == np.uint16:
        rc = lib.oracle_softmax_rows_bf16(_ptr(x), _ptr(out), rows, cols, ldx, ldy, threads)
    else:
        raise TypeError(f"unsupported dtype {x.dtype}")
    if rc != 0:
        raise ValueError("invalid softmax sizes")
    return out


# ------------------------------------------------------------- layernorm --
def layernorm_rows(x: np.ndarray, gamma: np.ndarray | None = None, beta: np.ndarray | None = None,
                   eps: float = 1e-5, gelu: bool = False, threads: int = 1) -> np.ndarray:
    """LayerNorm along the last axis of a 2-D array (float64, float32 or bf16 uint16).

    y = (x - mean) / sqrt(var + eps) * gamma + beta (biased variance), then
    tanh-GELU if ``gelu``; gamma and beta are per-column arrays of x's dtype
    or None. Computed in double, rounded once to the storage type.
    """
    if x.ndim != 2:
        raise ValueError("layernorm_rows expects a 2-D array")
    rows, cols = x.shape
    x = np.ascontiguousarray(x)
    out = np.empty((rows, cols), x.dtype)
    g = None if gamma is None else np.ascontiguousarray(gamma, x.dtype).ravel()
    b = None if beta is None else np.ascontiguousarray(beta, x.dtype).ravel()
    for a in (g, b):
        if a is not None and a.size != cols:
            raise ValueError("gamma and beta need one entry per column")
    gp = None if g is None else _ptr(g)
    bp = None if b is None else _ptr(b)
    lib = _load()
    if x.dtype == np.float64:
        rc = lib.oracle_layernorm_rows_f64(_ptr(x), _ptr(out), rows, cols, cols, cols, gp, bp,
                                           float(eps), int(gelu))
    elif x.dtype == np.float32:
        rc = lib.oracle_layernorm_rows_f32(_ptr(x), _ptr(out), rows, cols, cols, cols, gp, bp,
                                           float(eps), int(gelu), threads)
    elif x.dtype == np.uint16:
        rc = lib.oracle_layernorm_rows_bf16(_ptr(x), _ptr(out), rows, cols, cols, cols, gp, bp,
                                            float(eps), int(gelu), threads)
    else:
        raise TypeError(f"unsupported dtype {x.dtype}")
    if rc != 0:
        raise ValueError("invalid layernorm sizes or eps")
    return out


# -------------------------------------------------------------- backward --
def gelu_tanh_grad_f64(x: np.ndarray) -> np.ndarray:
    """GELU'(x) of the tanh form in double, unrounded."""
    x = _c(x, np.float64)
    y = np.empty_like(x)
    _load().oracle_gelu_tanh_grad_f64(_ptr(x), _ptr(y), x.size)
    return y


def gelu_tanh_backward(x: np.ndarray, dy: np.ndarray, threads: int = 1) -> np.ndarray:
    """dx = dy * GELU'(x) for fp32 (float32) or bf16 (uint16) data, same dtype out."""
    if x.shape != dy.shape or x.dtype != dy.dtype:
        raise ValueError("x and dy must match in shape and dtype")
    lib = _load()
    if x.dtype == np.uint16:
        x, dy = _c(x, np.uint16), _c(dy, np.uint16)
        dx = np.empty_like(x)
        lib.oracle_gelu_tanh_bwd_bf16(_ptr(x), _ptr(dy), _ptr(dx), x.size, threads)
        return dx
    x, dy = _c(x, np.float32), _c(dy, np.float32)
    dx = np.empty_like(x)
    lib.oracle_gelu_tanh_bwd_f32(_ptr(x), _ptr(dy), _ptr(dx), x.size, threads)
    return dx


def softmax_rows_backward(y: np.ndarray, dy: np.ndarray, threads: int = 1) -> np.ndarray:
    """dx_j = y_j (dy_j - sum_k y_k dy_k) per row (float64, float32 or bf16 uint16)."""
    if y.ndim != 2 or y.shape != dy.shape or y.dtype != dy.dtype:
        raise ValueError("y and dy must be 2-D arrays of one shape and dtype")
    rows, cols = y.shape
    y, dy = np.ascontiguousarray(y), np.ascontiguousarray(dy)
    dx = np.empty_like(y)
    lib = _load()
    if y.dtype == np.float64:
        rc = lib.oracle_softmax_bwd_rows_f64(_ptr(y), _ptr(dy), _ptr(dx), rows, cols)
    elif y.dtype == np.float32:
        rc = lib.oracle_softmax_bwd_rows_f32(_ptr(y), _ptr(dy), _ptr(dx), rows, cols, threads)
    elif y.dtype == np.uint16:
        rc = lib.oracle_softmax_bwd_rows_bf16(_ptr(y), _ptr(dy), _ptr(dx), rows, cols, threads)
    else:
        raise TypeError(f"unsupported dtype {y.dtype}")
    if rc != 0:
        raise ValueError("invalid sizes")
    return dx


# ------------------------------------------------------ linear + GELU -----
def _as_f64(a: np.ndarray) -> np.ndarray:
    return bf16_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)


def linear_gelu(x: np.ndarray, w: np.ndarray, bias: np.ndarray | None = None, gelu: bool = True,
                rows: np.ndarray | None = None, activation: str | None = None) -> np.ndarray:
    """y = act(x w^T + bias) in double, rounded once to x's storage type.

    act: tanh-GELU (gelu=True) or none, or the named ``activation`` ("none",
    "gelu_tanh", "relu": x > 0 ? x : +0 with NaN kept).

    x [M, K], w [N, K], bias [N] (float32, float16, or bf16 as uint16
    bits). The product is numpy's float64 matmul of the stored values (a
    library primitive used as one step); the bias is added in double, GELU
    is the oracle's real tanh-GELU; the result is rounded to fp32 and, for
    bf16 or fp16 data, then to that type (nearest even). ``rows`` selects a
    subset of rows of x (sampling).
    """
    xd = _as_f64(x if rows is None else x[np.asarray(rows)])
    wd = _as_f64(w)
    acc = xd @ wd.T
    if bias is not None:
        acc = acc + _as_f64(bias)[None, :]
    act = activation if activation is not None else ("gelu_tanh" if gelu else "none")
    if act == "gelu_tanh":
        acc = gelu_tanh_f64(acc).reshape(acc.shape)
    elif act == "relu":
        acc = np.where((acc > 0) | np.isnan(acc), acc, 0.0)
    elif act != "none":
        raise ValueError(f"unknown activation {act!r}")
    out = acc.astype(np.float32)
    if x.dtype == np.uint16:
        return f32_to_bf16(out).reshape(out.shape)
    return out.astype(np.float16) if x.dtype == np.float16 else out


def linear_abs_bound(x: np.ndarray, w: np.ndarray, rows: np.ndarray | None = None) -> np.ndarray:
    """(|x| |w|^T)_ij in double: the scale of the accumulation error bounds."""
    xd = np.abs(_as_f64(x if rows is None else x[np.asarray(rows)]))
    return xd @ np.abs(_as_f64(w)).T


# ------------------------------------------------------------- attention --
def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, causal: bool = True,
              rows: dict | None = None) -> np.ndarray:
    """O = softmax(Q K^T / sqrt(d) + mask) V per (batch, head), rounded once.

    q, k, v: [B, H, T, d] (float32, float16, or bf16 as uint16 bits). The
    causal mask keeps key j for query i when j <= i ("Lecture 6: GPU Kernels
    and Triton", section 8: the mask q_offset >= kv_offset). Scores and the
    products use numpy's float64 matmul (a library step); the row softmax is
    the oracle's own (max, exponentials, sum, normalise, in double); the
    result is rounded to fp32 and, for bf16 or fp16 data, then to that type
    (nearest even). ``rows`` maps (b, h)
    to an array of query indices to compute only those rows (sampling);
    then the result is {(b, h): [len(rows), d]}.
    """
    Bn, Hn, T, d = q.shape
    scale = 1.0 / np.sqrt(d)

    def one(b, h, qi):
        qd = _as_f64(q[b, h][qi])
        kd = _as_f64(k[b, h])
        vd = _as_f64(v[b, h])
        sc = (qd @ kd.T) * scale
        if causal:
            sc = np.where(np.arange(T)[None, :] <= np.asarray(qi)[:, None], sc, -np.inf)
        pr = softmax_rows(np.ascontiguousarray(sc))
        o = (pr @ vd).astype(np.float32)
        if q.dtype == np.uint16:
            return f32_to_bf16(o).reshape(o.shape)
        return o.astype(np.float16) if q.dtype == np.float16 else o

    if rows is not None:
        return {key: one(key[0], key[1], np.asarray(idx)) for key, idx in rows.items()}
    out = np.empty(q.shape, q.dtype)
    for b in range(Bn):
        for h in range(Hn):
            out[b, h] = one(b, h, np.arange(T))
    return out
