"""AddressSanitizer + UndefinedBehaviorSanitizer builds (CPU only).

* The oracle (oracle/oracle.cpp), built with g++ -fsanitize=address,undefined
  next to tests/sanitize/oracle_check.cpp, which runs every oracle entry
  point over special values, strided rows, odd sizes and more threads than
  elements.
* The library's host code: every source of libfusedops compiled by hipcc
  with the sanitizers on the host pass only (-Xarch_host before each
  -fsanitize=; the gfx950 device code is built as usual and never runs
  here), linked with tests/sanitize/api_check.cpp, which calls every entry
  point with extreme sizes, strides and pointers. All of those calls are
  refused by the host checks before any HIP call.

Any sanitizer report aborts the driver (-fno-sanitize-recover=all), so a
zero exit status and the driver's "ok" mean a clean run.
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
HERE = Path(__file__).resolve().parent / "sanitize"
CSRC = ROOT / "memory_bound_elementwise_fk_amd" / "csrc"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["api.hip", "elementwise.hip", "softmax.hip", "layernorm.hip", "backward.hip",
           "gemm.hip", "attention.hip"]
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all"]
RUN_ENV = {**os.environ, "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
           "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"}


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(map(str, cmd))}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = tmp_path / "oracle_check"
    _run(["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
          *SAN, str(ROOT / "oracle" / "oracle.cpp"), str(HERE / "oracle_check.cpp"),
          "-o", str(exe), "-lpthread"])
    r = _run([str(exe)], env=RUN_ENV, timeout=120)
    assert r.stdout.strip().endswith("ok")


@pytest.mark.skipif(not Path(HIPCC).exists(), reason="hipcc not available")
def test_library_host_checks_under_asan_ubsan(tmp_path):
    host_san = [f for flag in SAN for f in ("-Xarch_host", flag)]

    def compile_one(src):
        obj = tmp_path / (Path(src).stem + ".o")
        _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
              "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              *host_san, f"-I{ROOT / 'include'}", "-c", str(CSRC / src), "-o", str(obj)])
        return obj

    drv = tmp_path / "api_check.o"
    _run(["g++", "-std=c++17", "-O1", "-g", *SAN, f"-I{ROOT / 'include'}", "-c",
          str(HERE / "api_check.cpp"), "-o", str(drv)])
    jobs = max(1, min(8, len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(jobs) as pool:
        objs = list(pool.map(compile_one, SOURCES))
    exe = tmp_path / "api_check"
    _run(["g++", *SAN, str(drv), *map(str, objs), "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib", "-o", str(exe)])
    r = _run([str(exe)], env=RUN_ENV, timeout=300)
    assert r.stdout.strip().endswith("ok")
