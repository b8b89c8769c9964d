"""Pins for the tile/mask model and the byte accounting (CPU only).

* The Triton tutorial page's worked example: 7 elements, BLOCK_SIZE 3 ->
  3 programs covering {0,1,2}, {3,4,5}, {6}; program 2 has offsets
  [6, 7, 8] and mask [1, 0, 0] (tests/golden/masking_worked_example.json).
* Brute force: for every n and block size the masked offsets cover
  [0, n) exactly once.
* The fusion traffic figure of "Lecture 6: GPU Kernels and Triton",
  section 1.1: three ops over 32 MB move 192 MB unfused and 64 MB fused
  (tests/golden/fusion_traffic.json); the benchmark's byte accounting for
  the chain workload must reproduce it.
"""
import json
from pathlib import Path

import pytest

from memory_bound_elementwise_fk_amd import workloads
from oracle import tiling

GOLDEN = Path(__file__).parent / "golden"


def test_worked_masking_example():
    g = json.loads((GOLDEN / "masking_worked_example.json").read_text())
    progs = tiling.programs(g["n_elements"], g["block_size"])
    assert len(progs) == g["grid"] == tiling.cdiv(7, 3)
    for (pid, offs, mask), want in zip(progs, g["programs"]):
        assert pid == want["pid"]
        assert [o for o, m in zip(offs, mask) if m] == want["elements"]
        if "offsets" in want:
            assert offs == want["offsets"]
            assert mask == want["mask"]


def test_masked_offsets_cover_each_element_once():
    for n in range(0, 130):
        for block in range(1, 19):
            cov = tiling.covered(n, block)
            assert cov == list(range(n))
            assert len(tiling.programs(n, block)) == -(-n // block)


def test_cdiv_rejects_bad_arguments():
    with pytest.raises(ValueError):
        tiling.cdiv(5, 0)
    with pytest.raises(ValueError):
        tiling.cdiv(-1, 3)


def test_fusion_traffic_figure():
    g = json.loads((GOLDEN / "fusion_traffic.json").read_text())
    w = workloads.WORKLOADS["C3"]
    assert w.numel * w.esize == g["tensor_bytes"]
    assert workloads.algorithmic_bytes("C3") == g["fused_bytes"]
    assert workloads.algorithmic_bytes("C3", unfused=True) == g["unfused_bytes"]
    assert g["unfused_bytes"] // g["fused_bytes"] == g["ratio"]


def test_algorithmic_bytes_per_workload():
    assert workloads.algorithmic_bytes("C1") == 8_000_024
    assert workloads.algorithmic_bytes("C2") == 32_768_000
    assert workloads.algorithmic_bytes("C4") == 536_870_912
    assert workloads.algorithmic_bytes("C5a") == 1_073_741_824
    assert workloads.algorithmic_bytes("C5b") == 4_294_967_296
