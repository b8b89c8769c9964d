"""M0 in the kernels that issue direct global-to-LDS loads from inline asm
(CPU only: builds the device code to gfx950 assembly and reads it).

The Linear and attention kernels write M0 inside an asm statement that also
issues the global_load_lds_dwordx4 reading it (csrc/gemm_kernels.hpp,
lds_dma16). That is only sound while nothing else in those kernels keeps a
value in M0: the compiler would not expect the asm to change it. This test
checks the built code for exactly that: every instruction that names m0 is
an `s_mov_b32 m0, sN` immediately followed by the direct load, and no
instruction that reads M0 implicitly (relative register moves, LDS-direct,
GWS/ordered-count LDS ops, messages) appears.
"""
import re
import subprocess
from pathlib import Path

import pytest

from memory_bound_elementwise_fk_amd import build as fkbuild

# instructions that use M0 without naming it
IMPLICIT_M0 = re.compile(r"^\s*(s_movrel|v_movrel|s_sendmsg|ds_gws|ds_ordered|ds_append|"
                         r"ds_consume|v_interp|s_setreg_b32\s+hwreg\(HW_REG_LDS)")


def _asm(source: str, tmp_path: Path) -> list[str]:
    out = tmp_path / (source + ".s")
    flags = [f for f in fkbuild.FLAGS if f != "-fPIC"]
    cmd = [fkbuild.HIPCC, *flags, f"-I{fkbuild.INCLUDE}", "--cuda-device-only", "-S", "-o",
           str(out), str(fkbuild.CSRC / source)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    if r.returncode != 0:
        pytest.fail(f"hipcc failed on {source}:\n{r.stderr[-2000:]}")
    return out.read_text().splitlines()


def _instructions(lines):
    """(index, text) of instruction lines, comments and directives dropped."""
    for i, line in enumerate(lines):
        t = line.split(";")[0].strip()
        if not t or t.startswith(".") or t.endswith(":"):
            continue
        yield i, t


@pytest.mark.parametrize("source", ["gemm.hip", "attention.hip"])
def test_m0_is_written_only_for_the_direct_loads(source, tmp_path):
    if not Path(fkbuild.HIPCC).exists():
        pytest.skip("hipcc not available")
    insts = list(_instructions(_asm(source, tmp_path)))
    writes = 0
    for n, (i, t) in enumerate(insts):
        assert not IMPLICIT_M0.match(t), f"{source}:{i}: instruction reading M0: {t}"
        if not re.search(r"\bm0\b", t):
            continue
        assert re.fullmatch(r"s_mov_b32\s+m0,\s*s\d+", t), f"{source}:{i}: other use of m0: {t}"
        nxt = insts[n + 1][1] if n + 1 < len(insts) else ""
        assert nxt.startswith("global_load_lds_dwordx4"), (
            f"{source}:{i}: m0 written but not read by the next instruction ({nxt})")
        writes += 1
    assert writes > 0, f"{source}: no direct loads found (the check would be vacuous)"
