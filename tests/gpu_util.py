"""Helpers of the GPU parity tests: guarded device buffers and transfers."""
import numpy as np
import torch

from memory_bound_elementwise_fk_amd import workloads as wl

DEV = "cuda:0"
GUARD = 1024  # canary elements on each side of an output
# NaN bit patterns no kernel writes: fp32 0x7FC0DEAD, bf16 0x7FC1
CANARY = {torch.float32: (torch.int32, 0x7FC0DEAD), torch.bfloat16: (torch.int16, 0x7FC1)}
CANARY_BITS = {"f32": 0x7FC0DEAD, "bf16": 0x7FC1}


def tdtype(dt: str):
    return torch.float32 if dt == "f32" else torch.bfloat16


def np_dtype(dt: str):
    return np.float32 if dt == "f32" else np.uint16


def guarded(shape, dtype):
    """(full, view): a device buffer filled with canaries and the inner view."""
    n = int(np.prod(shape))
    full = torch.empty(n + 2 * GUARD, dtype=dtype, device=DEV)
    idt, val = CANARY[dtype]
    full.view(idt).fill_(val)
    return full, full[GUARD:GUARD + n].view(shape)


def guards_intact(full, n: int) -> bool:
    idt, val = CANARY[full.dtype]
    bits = full.view(idt)
    return bool((bits[:GUARD] == val).all() and (bits[GUARD + n:] == val).all())


def to_dev(a: np.ndarray):
    return wl.to_torch(np.ascontiguousarray(a), DEV)


def to_host(t) -> np.ndarray:
    torch.cuda.synchronize()
    return wl.from_torch(t)


def random_input(shape, dt: str, scale: float, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    return x if dt == "f32" else wl.f32_to_bf16_bits(x).reshape(shape)
