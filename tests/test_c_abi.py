"""The C ABI from plain C (CPU only): tests/c_abi_check.c includes
include/fusedops.h as C99, links libfusedops.so and checks the pure host
queries and argument errors (no call in it reaches the GPU)."""
import shutil
import subprocess

import pytest

import memory_bound_elementwise_fk_amd as fk
from tests.test_abi import ROOT


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_header_compiles_as_c99_and_library_links_from_c(tmp_path):
    if not fk.LIB_PATH.exists():
        from memory_bound_elementwise_fk_amd.build import build

        build()
    libdir = fk.LIB_PATH.parent
    exe = tmp_path / "c_abi_check"
    cc = subprocess.run(
        ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
         "-I", str(ROOT / "include"), str(ROOT / "tests" / "c_abi_check.c"),
         "-L", str(libdir), "-lfusedops", f"-Wl,-rpath,{libdir}", "-o", str(exe)],
        capture_output=True, text=True, timeout=120)
    assert cc.returncode == 0, cc.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert run.stdout.strip() == "ok"
