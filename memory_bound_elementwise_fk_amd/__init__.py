"""Python binding of libfusedops (fused memory-bound kernels for MI355X).

Argument marshalling only: every function forwards torch device tensors'
pointers, sizes and strides, plus the current HIP stream, to the C entry
point of the same name in ``libfusedops.so`` (declared in
``include/fusedops.h``); all computation happens in the HIP kernels. There
is no fallback: without the built library every call raises.

Tensors must live on a GPU device; torch is used only for device memory and
streams. ``y`` is written in place (``y`` may be ``x`` itself).
"""
from __future__ import annotations

import contextlib
import ctypes
from pathlib import Path

LIB_PATH = Path(__file__).resolve().parent / "libfusedops.so"

FK_F32 = 0
FK_BF16 = 1
FK_F16 = 2  # fk_linear_gelu and fk_attention_fwd only
FK_OK = 0
FK_ERR_INVALID_ARG = -1
FK_ERR_UNSUPPORTED = -2
FK_ERR_OVERLAP = -3
FK_ERR_HIP = -4
FK_OP_ADD_SCALAR = 1
FK_OP_MUL_SCALAR = 2
FK_OP_GELU_TANH = 3
FK_OP_RELU = 4
FK_PATH_NONE = 0
FK_PATH_ONCHIP = 1
FK_PATH_SPLIT = 2
FK_PATH_ONLINE = 3
FK_ACT_NONE = 0
FK_ACT_GELU_TANH = 1
FK_ACT_RELU = 2
_ACTS = {"none": FK_ACT_NONE, "gelu_tanh": FK_ACT_GELU_TANH, "relu": FK_ACT_RELU}
FK_MAX_OPS = 8
FK_SOFTMAX_SCRATCH_BYTES = 1 << 20

__all__ = [
    "FusedOpsError", "lib", "fk_gelu_tanh", "fk_elementwise_chain", "fk_softmax_rows",
    "fk_softmax_rows_online", "fk_softmax_rows_ws", "fk_softmax_workspace_bytes",
    "fk_softmax_rows_path", "fk_softmax_rows_noalloc", "FK_SOFTMAX_SCRATCH_BYTES",
    "fk_set_split_wait_limit", "fk_softmax_onchip_max_cols", "fk_layernorm_rows",
    "fk_layernorm_max_cols", "fk_copy", "fk_status_string", "layernorm_rows",
    "fk_gelu_tanh_backward", "fk_softmax_rows_backward", "fk_softmax_backward_max_cols",
    "gelu_tanh_backward", "softmax_rows_backward", "fk_linear_gelu", "linear_gelu",
    "fk_attention_fwd", "attention_fwd",
    "gelu_tanh", "elementwise_chain", "softmax_rows",
]


class FusedOpsError(RuntimeError):
    """A libfusedops entry point returned a negative fk_status."""

    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {fk_status_string(status)} (status {status})")
        self.status = status


class fk_op(ctypes.Structure):  # noqa: N801  (C name)
    _fields_ = [("kind", ctypes.c_int32), ("scalar", ctypes.c_float)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library with argument types set (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not LIB_PATH.exists():
        raise RuntimeError(
            f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc, gfx950)")
    L = ctypes.CDLL(str(LIB_PATH))
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.fk_gelu_tanh.argtypes = [vp, vp, i64, i32, vp]
    L.fk_gelu_tanh.restype = i32
    L.fk_elementwise_chain.argtypes = [vp, vp, i64, i32, ctypes.POINTER(fk_op), i32, vp]
    L.fk_elementwise_chain.restype = i32
    for name in ("fk_softmax_rows", "fk_softmax_rows_online"):
        fn = getattr(L, name)
        fn.argtypes = [vp, vp, i64, i64, i64, i64, i32, vp]
        fn.restype = i32
    L.fk_softmax_rows_ws.argtypes = [vp, vp, i64, i64, i64, i64, i32, vp, i64, vp]
    L.fk_softmax_rows_ws.restype = i32
    L.fk_softmax_rows_noalloc.argtypes = [vp, vp, i64, i64, i64, i64, i32, vp]
    L.fk_softmax_rows_noalloc.restype = i32
    L.fk_softmax_rows_path.argtypes = [vp, vp, i64, i64, i64, i64, i32, i64]
    L.fk_softmax_rows_path.restype = i32
    L.fk_softmax_workspace_bytes.argtypes = [i64, i64, i32]
    L.fk_softmax_workspace_bytes.restype = i64
    L.fk_set_split_wait_limit.argtypes = [i64]
    L.fk_set_split_wait_limit.restype = i64
    L.fk_layernorm_rows.argtypes = [vp, vp, i64, i64, i64, i64, vp, vp, ctypes.c_float, i32, i32,
                                    vp]
    L.fk_layernorm_rows.restype = i32
    L.fk_gelu_tanh_backward.argtypes = [vp, vp, vp, i64, i32, vp]
    L.fk_gelu_tanh_backward.restype = i32
    L.fk_softmax_rows_backward.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, i32, vp]
    L.fk_softmax_rows_backward.restype = i32
    L.fk_softmax_backward_max_cols.argtypes = [i32]
    L.fk_softmax_backward_max_cols.restype = i64
    L.fk_linear_gelu.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i32, i32, vp]
    L.fk_linear_gelu.restype = i32
    L.fk_attention_fwd.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, ctypes.POINTER(i64), i32,
                                   i32, vp]
    L.fk_attention_fwd.restype = i32
    L.fk_layernorm_max_cols.argtypes = [i32]
    L.fk_layernorm_max_cols.restype = i64
    L.fk_softmax_onchip_max_cols.argtypes = [i32]
    L.fk_softmax_onchip_max_cols.restype = i64
    L.fk_copy.argtypes = [vp, vp, i64, vp]
    L.fk_copy.restype = i32
    L.fk_status_string.argtypes = [i32]
    L.fk_status_string.restype = ctypes.c_char_p
    _lib = L
    return L


def fk_status_string(status: int) -> str:
    return lib().fk_status_string(int(status)).decode()


# ------------------------------------------------------------ marshalling -
# These run on every call, so they keep to cheap tensor properties: a short
# launch (attention at T = 128 takes 8.5 us on the device) is otherwise
# bound by the host's argument checks.
_torch_mod = None
_dtype_codes = None
_raw_stream = None


def _torch():
    global _torch_mod, _dtype_codes, _raw_stream
    if _torch_mod is None:
        import torch

        _dtype_codes = {torch.float32: FK_F32, torch.bfloat16: FK_BF16, torch.float16: FK_F16}
        # the current stream's handle for a device index, without building a
        # torch.cuda.Stream object per call (that costs ~2 us)
        _raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        _torch_mod = torch
    return _torch_mod


def _dtype_code(t) -> int:
    _torch()
    code = _dtype_codes.get(t.dtype)
    if code is None:  # FK_F16 is refused by the library outside Linear and attention
        raise TypeError(f"unsupported dtype {t.dtype} (float32, bfloat16, or float16 for Linear and attention)")
    return code


def _device_tensor(t, name: str):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor, got device {t.device}")


def _on_device(t):
    """Context making t's GPU current for the call: a no-op when it already
    is (entering torch.cuda.device costs a few microseconds per call)."""
    torch = _torch()
    if t.get_device() == torch.cuda.current_device():
        return contextlib.nullcontext()
    return torch.cuda.device(t.device)


def _stream_handle(t, stream) -> int | None:
    if stream is None:
        torch = _torch()
        if _raw_stream is not None:
            return _raw_stream(t.get_device())
        return torch.cuda.current_stream(t.device).cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _check(rc: int, what: str) -> None:
    if rc != FK_OK:
        raise FusedOpsError(rc, what)


def _flat_pair(x, y, what: str):
    _device_tensor(x, "x")
    _device_tensor(y, "y")
    if x.dtype != y.dtype:
        raise TypeError(f"{what}: x and y dtypes differ")
    if x.numel() != y.numel():
        raise ValueError(f"{what}: x has {x.numel()} elements, y {y.numel()}")
    if x.device != y.device:
        raise ValueError(f"{what}: x and y on different devices")
    if not (x.is_contiguous() and y.is_contiguous()):
        raise ValueError(f"{what}: x and y must be contiguous")
    return x.numel(), _dtype_code(x)


def _ops_array(ops):
    ops = list(ops)
    arr = (fk_op * max(1, len(ops)))()
    for i, (kind, scalar) in enumerate(ops):
        arr[i].kind = int(kind)
        arr[i].scalar = float(scalar)
    return arr, len(ops)


def _rows_pair(x, y, what: str):
    _device_tensor(x, "x")
    _device_tensor(y, "y")
    if x.dtype != y.dtype:
        raise TypeError(f"{what}: x and y dtypes differ")
    if x.dim() != 2 or y.dim() != 2 or tuple(x.shape) != tuple(y.shape):
        raise ValueError(f"{what}: x and y must be 2-D of the same shape")
    if x.device != y.device:
        raise ValueError(f"{what}: x and y on different devices")
    rows, cols = x.shape
    if cols > 1 and (x.stride(1) != 1 or y.stride(1) != 1):
        raise ValueError(f"{what}: rows must be contiguous (unit column stride)")
    ldx = x.stride(0) if rows > 1 else cols
    ldy = y.stride(0) if rows > 1 else cols
    return rows, cols, ldx, ldy, _dtype_code(x)


# -------------------------------------------------------- entry points ----
def fk_gelu_tanh(x, y, stream=None) -> None:
    """y = tanh-GELU(x) elementwise (fp32 or bf16, contiguous, same size)."""
    n, dt = _flat_pair(x, y, "fk_gelu_tanh")
    with _on_device(x):
        _check(lib().fk_gelu_tanh(x.data_ptr(), y.data_ptr(), n, dt, _stream_handle(x, stream)),
               "fk_gelu_tanh")


def fk_elementwise_chain(x, y, ops, stream=None) -> None:
    """y = ops applied in order to x; ops is a sequence of (kind, scalar)."""
    n, dt = _flat_pair(x, y, "fk_elementwise_chain")
    arr, count = _ops_array(ops)
    with _on_device(x):
        _check(lib().fk_elementwise_chain(x.data_ptr(), y.data_ptr(), n, dt, arr, count,
                                          _stream_handle(x, stream)), "fk_elementwise_chain")


def fk_softmax_rows(x, y, stream=None) -> None:
    """Softmax along each row of a 2-D x into y (row strides honoured)."""
    rows, cols, ldx, ldy, dt = _rows_pair(x, y, "fk_softmax_rows")
    with _on_device(x):
        _check(lib().fk_softmax_rows(x.data_ptr(), y.data_ptr(), rows, cols, ldx, ldy, dt,
                                     _stream_handle(x, stream)), "fk_softmax_rows")


def fk_softmax_rows_online(x, y, stream=None) -> None:
    """As fk_softmax_rows, always through the online two-pass kernel."""
    rows, cols, ldx, ldy, dt = _rows_pair(x, y, "fk_softmax_rows_online")
    with _on_device(x):
        _check(lib().fk_softmax_rows_online(x.data_ptr(), y.data_ptr(), rows, cols, ldx, ldy, dt,
                                            _stream_handle(x, stream)), "fk_softmax_rows_online")


def fk_softmax_rows_ws(x, y, workspace, stream=None) -> None:
    """As fk_softmax_rows with a caller-owned workspace (a device tensor of
    at least fk_softmax_workspace_bytes bytes, any contents; None when that
    is 0)."""
    rows, cols, ldx, ldy, dt = _rows_pair(x, y, "fk_softmax_rows_ws")
    if workspace is None:
        wptr, wbytes = None, 0
    else:
        _device_tensor(workspace, "workspace")
        wptr, wbytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    with _on_device(x):
        _check(lib().fk_softmax_rows_ws(x.data_ptr(), y.data_ptr(), rows, cols, ldx, ldy, dt,
                                        wptr, wbytes, _stream_handle(x, stream)),
               "fk_softmax_rows_ws")


def _dtype_arg(dtype) -> int:
    if isinstance(dtype, int):
        return dtype
    torch = _torch()
    return {torch.float32: FK_F32, torch.bfloat16: FK_BF16, torch.float16: FK_F16}.get(dtype, -1)


def fk_softmax_rows_noalloc(x, y, stream=None) -> None:
    """As fk_softmax_rows_ws, with the library's static device scratch as the
    split path's workspace: no allocation at all (FusedOpsError with
    FK_ERR_UNSUPPORTED when the shape needs more than
    FK_SOFTMAX_SCRATCH_BYTES)."""
    rows, cols, ldx, ldy, dt = _rows_pair(x, y, "fk_softmax_rows_noalloc")
    with _on_device(x):
        _check(lib().fk_softmax_rows_noalloc(x.data_ptr(), y.data_ptr(), rows, cols, ldx, ldy, dt,
                                             _stream_handle(x, stream)),
               "fk_softmax_rows_noalloc")


def fk_softmax_rows_path(x, y, workspace_bytes: int = 0) -> int:
    """FK_PATH_* of fk_softmax_rows_ws(x, y, <workspace of workspace_bytes>)
    (workspace_bytes = 0: the path of fk_softmax_rows). Host query only."""
    rows, cols, ldx, ldy, dt = _rows_pair(x, y, "fk_softmax_rows_path")
    v = lib().fk_softmax_rows_path(x.data_ptr(), y.data_ptr(), rows, cols, ldx, ldy, dt,
                                   int(workspace_bytes))
    if v < 0:
        raise FusedOpsError(int(v), "fk_softmax_rows_path")
    return int(v)


def fk_softmax_workspace_bytes(rows: int, cols: int, dtype) -> int:
    """Workspace bytes fk_softmax_rows_ws needs (0: none)."""
    v = lib().fk_softmax_workspace_bytes(int(rows), int(cols), _dtype_arg(dtype))
    if v < 0:
        raise FusedOpsError(int(v), "fk_softmax_workspace_bytes")
    return int(v)


def fk_set_split_wait_limit(polls: int) -> int:
    """Set the split path's bound on waiting polls; returns the previous bound."""
    v = lib().fk_set_split_wait_limit(int(polls))
    if v < 0:
        raise FusedOpsError(int(v), "fk_set_split_wait_limit")
    return int(v)


def fk_softmax_onchip_max_cols(dtype) -> int:
    """Widest row held on chip for a torch dtype or an FK_* code."""
    v = lib().fk_softmax_onchip_max_cols(_dtype_arg(dtype))
    if v < 0:
        raise FusedOpsError(int(v), "fk_softmax_onchip_max_cols")
    return int(v)


def _param(p, x, name: str):
    """Device pointer of an optional per-column parameter (None -> NULL)."""
    if p is None:
        return None
    _device_tensor(p, name)
    if p.dtype != x.dtype or p.dim() != 1 or p.numel() != x.shape[-1] or not p.is_contiguous():
        raise ValueError(f"{name} must be a contiguous 1-D tensor of x's dtype with one entry "
                         f"per column")
    if p.device != x.device:
        raise ValueError(f"{name} is on another device than x")
    return p.data_ptr()


def fk_layernorm_rows(x, y, gamma=None, beta=None, eps: float = 1e-5, gelu: bool = False,
                      stream=None) -> None:
    """LayerNorm along each row of a 2-D x into y (optionally then tanh-GELU)."""
    rows, cols, ldx, ldy, dt = _rows_pair(x, y, "fk_layernorm_rows")
    g, b = _param(gamma, x, "gamma"), _param(beta, x, "beta")
    with _on_device(x):
        _check(lib().fk_layernorm_rows(x.data_ptr(), y.data_ptr(), rows, cols, ldx, ldy, g, b,
                                       float(eps), int(bool(gelu)), dt, _stream_handle(x, stream)),
               "fk_layernorm_rows")


def fk_layernorm_max_cols(dtype) -> int:
    """Widest row fk_layernorm_rows accepts for a torch dtype or an FK_* code."""
    v = lib().fk_layernorm_max_cols(_dtype_arg(dtype))
    if v < 0:
        raise FusedOpsError(int(v), "fk_layernorm_max_cols")
    return int(v)


def fk_gelu_tanh_backward(x, dy, dx, stream=None) -> None:
    """dx = dy * GELU'(x) elementwise (fp32 or bf16, contiguous, same size)."""
    n, dt = _flat_pair(x, dx, "fk_gelu_tanh_backward")
    _flat_pair(dy, dx, "fk_gelu_tanh_backward")
    with _on_device(x):
        _check(lib().fk_gelu_tanh_backward(x.data_ptr(), dy.data_ptr(), dx.data_ptr(), n, dt,
                                           _stream_handle(x, stream)), "fk_gelu_tanh_backward")


def fk_softmax_rows_backward(y, dy, dx, stream=None) -> None:
    """dx = y * (dy - sum(y * dy)) per row of 2-D y, dy into dx (row strides honoured)."""
    rows, cols, ldy, lddx, dt = _rows_pair(y, dx, "fk_softmax_rows_backward")
    _, _, lddy, _, _ = _rows_pair(dy, dx, "fk_softmax_rows_backward")
    with _on_device(y):
        _check(lib().fk_softmax_rows_backward(y.data_ptr(), dy.data_ptr(), dx.data_ptr(), rows,
                                              cols, ldy, lddy, lddx, dt,
                                              _stream_handle(y, stream)),
               "fk_softmax_rows_backward")


def fk_softmax_backward_max_cols(dtype) -> int:
    """Widest row fk_softmax_rows_backward accepts for a torch dtype or an FK_* code."""
    v = lib().fk_softmax_backward_max_cols(_dtype_arg(dtype))
    if v < 0:
        raise FusedOpsError(int(v), "fk_softmax_backward_max_cols")
    return int(v)


def fk_linear_gelu(x, w, bias, y, gelu: bool = True, stream=None, activation: str | None = None
                   ) -> None:
    """y = act(x @ w.T + bias) for 2-D bf16/fp16 x [M, K], w [N, K], bias [N] or None, y [M, N].

    act is tanh-GELU (gelu=True) or none (gelu=False), or the named
    ``activation`` ("none", "gelu_tanh", "relu") when given."""
    for t, name in ((x, "x"), (w, "w"), (y, "y")):
        _device_tensor(t, name)
        if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
            raise ValueError(f"fk_linear_gelu: {name} must be 2-D with contiguous rows")
    M, K = x.shape
    N = w.shape[0]
    if w.shape[1] != K or tuple(y.shape) != (M, N):
        raise ValueError("fk_linear_gelu: shapes x [M, K], w [N, K], y [M, N] do not match")
    if x.dtype != w.dtype or x.dtype != y.dtype:
        raise TypeError("fk_linear_gelu: x, w and y must share a dtype")
    b = None
    if bias is not None:
        _device_tensor(bias, "bias")
        if bias.dtype != x.dtype or bias.dim() != 1 or bias.numel() != N or not bias.is_contiguous():
            raise ValueError("fk_linear_gelu: bias must be a contiguous [N] tensor of x's dtype")
        b = bias.data_ptr()
    if activation is None:
        act = FK_ACT_GELU_TANH if gelu else FK_ACT_NONE
    elif activation in _ACTS:
        act = _ACTS[activation]
    else:
        raise ValueError(f"fk_linear_gelu: activation must be one of {sorted(_ACTS)}")
    ld = lambda t, n: t.stride(0) if t.shape[0] > 1 else n  # noqa: E731
    with _on_device(x):
        _check(lib().fk_linear_gelu(x.data_ptr(), w.data_ptr(), b, y.data_ptr(), M, N, K,
                                    ld(x, K), ld(w, K), ld(y, N), act,
                                    _dtype_code(x), _stream_handle(x, stream)), "fk_linear_gelu")


def fk_attention_fwd(q, k, v, o, causal: bool = True, stream=None) -> None:
    """o = softmax(q k^T / sqrt(d) + mask) v for 4-D [B, H, T, d] tensors (any strides,
    contiguous head dimension)."""
    strides = []
    for t, name in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _device_tensor(t, name)
        if t.dim() != 4 or t.shape != q.shape:
            raise ValueError(f"fk_attention_fwd: {name} must be 4-D [B, H, T, d] like q")
        ts = t.stride()
        if t.shape[3] > 1 and ts[3] != 1:
            raise ValueError(f"fk_attention_fwd: {name} needs a contiguous head dimension")
        if t.dtype != q.dtype:
            raise TypeError("fk_attention_fwd: q, k, v, o must share a dtype")
        strides += ts[:3]
    B, H, T, d = q.shape
    st = (ctypes.c_int64 * 12)(*strides)
    with _on_device(q):
        _check(lib().fk_attention_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), B,
                                      H, T, d, st, int(bool(causal)), _dtype_code(q),
                                      _stream_handle(q, stream)), "fk_attention_fwd")


def fk_copy(x, y, nbytes: int | None = None, stream=None) -> None:
    """Copy nbytes (default: all of x) from x to y on the device."""
    _device_tensor(x, "x")
    _device_tensor(y, "y")
    if nbytes is None:
        nbytes = x.numel() * x.element_size()
    if nbytes > x.numel() * x.element_size() or nbytes > y.numel() * y.element_size():
        raise ValueError("fk_copy: nbytes exceeds a buffer")
    with _on_device(x):
        _check(lib().fk_copy(x.data_ptr(), y.data_ptr(), nbytes, _stream_handle(x, stream)),
               "fk_copy")


# ---------------------------------------------- allocating conveniences --
def gelu_tanh(x, stream=None):
    y = _torch().empty_like(x, memory_format=_torch().contiguous_format)
    fk_gelu_tanh(x, y, stream)
    return y


def elementwise_chain(x, ops, stream=None):
    y = _torch().empty_like(x, memory_format=_torch().contiguous_format)
    fk_elementwise_chain(x, y, ops, stream)
    return y


def softmax_rows(x, stream=None):
    y = _torch().empty(x.shape, dtype=x.dtype, device=x.device)
    fk_softmax_rows(x, y, stream)
    return y


def layernorm_rows(x, gamma=None, beta=None, eps: float = 1e-5, gelu: bool = False, stream=None):
    y = _torch().empty(x.shape, dtype=x.dtype, device=x.device)
    fk_layernorm_rows(x, y, gamma, beta, eps, gelu, stream)
    return y


def gelu_tanh_backward(x, dy, stream=None):
    dx = _torch().empty_like(x, memory_format=_torch().contiguous_format)
    fk_gelu_tanh_backward(x, dy, dx, stream)
    return dx


def softmax_rows_backward(y, dy, stream=None):
    dx = _torch().empty(y.shape, dtype=y.dtype, device=y.device)
    fk_softmax_rows_backward(y, dy, dx, stream)
    return dx


def linear_gelu(x, w, bias=None, gelu: bool = True, stream=None, activation: str | None = None):
    y = _torch().empty((x.shape[0], w.shape[0]), dtype=x.dtype, device=x.device)
    fk_linear_gelu(x, w, bias, y, gelu, stream, activation)
    return y


def attention_fwd(q, k, v, causal: bool = True, stream=None):
    o = _torch().empty(q.shape, dtype=q.dtype, device=q.device)
    fk_attention_fwd(q, k, v, o, causal, stream)
    return o
