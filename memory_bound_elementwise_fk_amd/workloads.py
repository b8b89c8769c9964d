"""Seeded synthetic inputs and byte accounting for the five workloads.

This module holds none of the method's arithmetic (no GELU, no softmax, no
rounding rule of its own): it draws random numbers and stores them in the
I/O dtype. It is the only code that both the HIP path's tests/benchmark and
the CPU oracle use.

Generator recipe (stated once, used everywhere):
  * values come in chunks of 2**22 elements; chunk ``k`` of stream ``s``
    for seed ``seed`` uses numpy's PCG64 seeded with
    ``SeedSequence([seed, s, k])``, so any chunk can be drawn on its own
    and the result does not depend on the thread count;
  * normals are numpy's ``standard_normal`` in float64, uniforms its
    ``random`` in float64; scaling and shifts are applied in float64;
  * the float64 value is rounded once to float32 (numpy ``astype``, nearest
    even); bf16 inputs are then rounded from that float32 by torch's
    float32 -> bfloat16 conversion (nearest even) and kept as uint16 bits.

Workloads (sizes and distributions of the pages' examples as configured):
  C1  tanh-GELU fp32, n = 1,000,003, x ~ N(0, 1), seed 0
  C2  softmax fp32, 4096 x 1000, x ~ N(0, 3^2), rows r % 16 == 0 get +80
  C3  chain fp32 y = 0.5 * GELU(x + 1), n = 8,388,608, x ~ U(-6, 6)
  C4  softmax bf16, 32768 x 4096, x ~ 8 * N(0, 1); each entry independently
      (probability 0.01, stream 1) replaced by bf16(-1e4) = -9984
  C5a softmax fp32, 1024 x 131072, x ~ N(0, 2^2)
  C5b tanh-GELU bf16, n = 2**30, x ~ N(0, 1)
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

CHUNK = 1 << 22
BF16_MINUS_1E4 = 0xC61C  # bf16(-1e4) = -9984, nearest even

OP_ADD_SCALAR = 1
OP_MUL_SCALAR = 2
OP_GELU_TANH = 3
CHAIN_C3 = ((OP_ADD_SCALAR, 1.0), (OP_GELU_TANH, 0.0), (OP_MUL_SCALAR, 0.5))


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str        # "gelu" | "chain" | "softmax"
    dtype: str       # "f32" | "bf16"
    shape: tuple     # (n,) or (rows, cols)
    dist: str        # "normal" | "uniform"
    scale: float     # sigma, or half-width for uniform
    seed: int = 0
    description: str = ""

    @property
    def numel(self) -> int:
        return int(np.prod(self.shape))

    @property
    def esize(self) -> int:
        return 4 if self.dtype == "f32" else 2


WORKLOADS = {
    "C1": Workload("C1", "gelu", "f32", (1_000_003,), "normal", 1.0,
                   description="tanh-GELU fp32 n=1,000,003 x~N(0,1)"),
    "C2": Workload("C2", "softmax", "f32", (4096, 1000), "normal", 3.0,
                   description="softmax fp32 4096x1000 x~N(0,9), every 16th row +80"),
    "C3": Workload("C3", "chain", "f32", (8_388_608,), "uniform", 6.0,
                   description="chain 0.5*GELU(x+1) fp32 n=8,388,608 x~U(-6,6)"),
    "C4": Workload("C4", "softmax", "bf16", (32768, 4096), "normal", 8.0,
                   description="softmax bf16 32768x4096 x~8N(0,1), 1% = -1e4"),
    "C5a": Workload("C5a", "softmax", "f32", (1024, 131072), "normal", 2.0,
                    description="wide-row softmax fp32 1024x131072 x~N(0,4)"),
    "C5b": Workload("C5b", "gelu", "bf16", (1 << 30,), "normal", 1.0,
                    description="tanh-GELU bf16 n=2^30 x~N(0,1)"),
}


def _threads(threads: int | None) -> int:
    if threads is not None:
        return max(1, threads)
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    cap = os.environ.get("OMP_NUM_THREADS")
    if cap and cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, min(n, 16))


def _rng(seed: int, stream: int, chunk: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream, chunk])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Store float32 values as bf16 (torch's nearest-even conversion), uint16 bits."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def draw(n: int, *, seed: int, stream: int = 0, dist: str = "normal", scale: float = 1.0,
         row_len: int = 0, row_period: int = 0, row_shift: float = 0.0, dtype: str = "f32",
         first_chunk: int = 0, threads: int | None = None) -> np.ndarray:
    """Draw ``n`` values (chunks ``first_chunk``...) and store them in ``dtype``.

    ``dist="normal"``: scale * N(0, 1). ``dist="uniform"``: U(-scale, scale).
    With ``row_period``: flat index i lies in row i // row_len; rows with
    row % row_period == 0 get ``row_shift`` added (in float64).
    """
    out = np.empty(n, np.float32 if dtype == "f32" else np.uint16)
    nchunks = (n + CHUNK - 1) // CHUNK

    def one(k: int) -> None:
        lo = k * CHUNK
        hi = min(n, lo + CHUNK)
        g = _rng(seed, stream, first_chunk + k)
        if dist == "normal":
            v = g.standard_normal(hi - lo, dtype=np.float64) * scale
        elif dist == "uniform":
            v = g.random(hi - lo, dtype=np.float64) * (2.0 * scale) - scale
        else:
            raise ValueError(dist)
        if row_period:
            base = (first_chunk * CHUNK) + lo
            rows = (base + np.arange(hi - lo, dtype=np.int64)) // row_len
            v = v + np.where(rows % row_period == 0, row_shift, 0.0)
        f = v.astype(np.float32)
        out[lo:hi] = f if dtype == "f32" else f32_to_bf16_bits(f)

    _pool_map(one, nchunks, threads, uses_torch=(dtype != "f32"))
    return out


def _pool_map(fn, nchunks: int, threads: int | None, uses_torch: bool = False) -> None:
    """Run fn(k) for every chunk on a thread pool (torch kept to one thread meanwhile)."""
    prev = None
    if uses_torch:
        import torch

        prev = torch.get_num_threads()
        torch.set_num_threads(1)
    try:
        with ThreadPoolExecutor(_threads(threads)) as ex:
            list(ex.map(fn, range(nchunks)))
    finally:
        if prev is not None:
            import torch

            torch.set_num_threads(prev)


def bernoulli_mask(n: int, p: float, *, seed: int, stream: int,
                   threads: int | None = None) -> np.ndarray:
    """Independent Bernoulli(p) per element (uniform < p), chunked like ``draw``."""
    out = np.empty(n, np.bool_)
    nchunks = (n + CHUNK - 1) // CHUNK

    def one(k: int) -> None:
        lo = k * CHUNK
        hi = min(n, lo + CHUNK)
        out[lo:hi] = _rng(seed, stream, k).random(hi - lo, dtype=np.float64) < p

    _pool_map(one, nchunks, threads)
    return out


def make_input(name: str, threads: int | None = None, rows: int | None = None) -> np.ndarray:
    """The seeded input of workload ``name`` (fp32 float32 or bf16 uint16 bits).

    ``rows`` (softmax only) keeps the first ``rows`` rows, drawn exactly as
    in the full workload.
    """
    w = WORKLOADS[name]
    if w.kind == "softmax":
        r, c = w.shape
        r = r if rows is None else min(rows, r)
        n = r * c
        kw = {}
        if name == "C2":
            kw = dict(row_len=c, row_period=16, row_shift=80.0)
        x = draw(n, seed=w.seed, dist=w.dist, scale=w.scale, dtype=w.dtype, threads=threads, **kw)
        if name == "C4":
            m = bernoulli_mask(n, 0.01, seed=w.seed, stream=1, threads=threads)
            x[m] = BF16_MINUS_1E4
        return x.reshape(r, c)
    return draw(w.numel, seed=w.seed, dist=w.dist, scale=w.scale, dtype=w.dtype, threads=threads)


# ---------------------------------------------------------------- bytes ---
def algorithmic_bytes(name: str, unfused: bool = False) -> int:
    """HBM bytes the op must move at least: one read and one write per element.

    The unfused chain runs its three ops as three kernels through
    intermediates, so it moves three reads and three writes per element.
    """
    w = WORKLOADS[name]
    per = 2 * w.esize * w.numel
    if w.kind == "chain" and unfused:
        return 3 * per
    return per


def to_torch(a: np.ndarray, device: str = "cpu"):
    """numpy (float32 or uint16 bf16 bits) -> torch tensor of float32/bfloat16."""
    import torch

    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(a)
    return t.to(device) if device != "cpu" else t


def from_torch(t) -> np.ndarray:
    """torch float32/bfloat16 tensor -> numpy float32 or uint16 bits (on host)."""
    import torch

    t = t.detach().to("cpu")
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)
    return t.contiguous().numpy()
