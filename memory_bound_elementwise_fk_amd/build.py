"""Build step for libfusedops: hipcc, gfx950 only, in-tree shared library.

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
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def build(extra_flags: list[str] | None = None) -> Path:
    """Compile every source into libfusedops.so (atomically replaced)."""
    tmp = LIB.with_suffix(".so.tmp")
    cmd = [HIPCC, *FLAGS, *(extra_flags or []), f"-I{INCLUDE}",
           *[str(CSRC / s) for s in SOURCES], "-o", str(tmp)]
    subprocess.run(cmd, check=True)
    tmp.replace(LIB)
    return LIB


if __name__ == "__main__":
    print(build(sys.argv[1:]), file=sys.stderr)
