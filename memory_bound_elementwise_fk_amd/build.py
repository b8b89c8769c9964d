"""Build step for libfusedops: hipcc, gfx950 only, in-tree shared library.

Each source compiles to its own object (in parallel, at most 16 jobs), then
one link produces the library, replaced atomically.

Flags:
  -ffp-contract=off    every fp32 op rounds as written (chain ops stay
                       separately rounded; FMAs are only the explicit fmaf)
  -target-feature -packed-fp32-ops
                       no packed fp32 instructions are emitted
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
INCLUDE = ROOT / "include"
LIB = PKG / "libfusedops.so"
SOURCES = ["api.hip", "elementwise.hip", "softmax.hip", "layernorm.hip", "backward.hip",
           "gemm.hip", "attention.hip"]
HEADERS = ["device_common.hpp", "ew_kernels.hpp", "softmax_kernels.hpp", "layernorm_kernels.hpp",
           "backward_kernels.hpp", "gemm_kernels.hpp", "attention_kernels.hpp",
           "launch.hpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _jobs() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n, len(SOURCES)))


def build(extra_flags: list[str] | None = None) -> Path:
    """Compile every source into libfusedops.so (atomically replaced)."""
    extra = list(extra_flags or [])
    with tempfile.TemporaryDirectory(prefix="fkbuild_") as tmpdir:
        objs = [Path(tmpdir) / (Path(s).stem + ".o") for s in SOURCES]

        def compile_one(i: int) -> None:
            cmd = [HIPCC, *FLAGS, *extra, f"-I{INCLUDE}", "-c", str(CSRC / SOURCES[i]),
                   "-o", str(objs[i])]
            subprocess.run(cmd, check=True)

        with ThreadPoolExecutor(_jobs()) as pool:
            list(pool.map(compile_one, range(len(SOURCES))))
        tmp = LIB.with_suffix(".so.tmp")
        subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *map(str, objs),
                        "-o", str(tmp)], check=True)
        tmp.replace(LIB)
    return LIB


if __name__ == "__main__":
    print(build(sys.argv[1:]), file=sys.stderr)
