"""Build step for the CPU oracle (test infrastructure): g++ -> liboracle.so.

IEEE arithmetic is kept exact as written: no fast-math and no FMA
contraction, so every double operation rounds as the source says.
"""
from __future__ import annotations

import subprocess
import sys
from pathlib import Path

HERE = Path(__file__).resolve().parent
SRC = HERE / "oracle.cpp"
OUT = HERE / "liboracle.so"

FLAGS = [
    "-std=c++17", "-O2", "-fPIC", "-shared",
    "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra",
]


def build() -> Path:
    tmp = OUT.with_suffix(".so.tmp")
    cmd = ["g++", *FLAGS, str(SRC), "-o", str(tmp), "-lpthread"]
    subprocess.run(cmd, check=True)
    tmp.replace(OUT)
    return OUT


if __name__ == "__main__":
    print(build(), file=sys.stderr)
