"""Host-side logic of bench.py (CPU only): argument refusal and the
conversion of rocprofv3 FETCH_SIZE / WRITE_SIZE counters into HBM bytes per
launch (scaled by a calibration copy of known size)."""
import csv
import json
import subprocess
import sys

import pytest

import bench
from memory_bound_elementwise_fk_amd import workloads as wl


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, str(bench.ROOT / "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_refuses_bad_step_counts():
    for args in (["--steps", "0"], ["--warmup", "-1"]):
        r = subprocess.run([sys.executable, str(bench.ROOT / "bench.py"), *args],
                           capture_output=True, text=True, timeout=120)
        assert r.returncode == 2, args


# rocprofv3 kernel names of the counted dispatches (fragments bench.py matches)
NAMES = {
    "copy": "void fk::copy_vec_kernel<64, 1, true>(unsigned int __vector(4) const*, ...)",
    "C3": "void fk::ew_vec_kernel<fk::IoF32, 64, 1, true, false, fk::AffActAffOp<1, 3, 2> >(...)",
    "C4": "void fk::softmax_reg_kernel<fk::IoBF16, 2, 4, true, true, 2>(...)",
    "C5a": "void fk::softmax_split_kernel<fk::IoF32, 256, 8, true, true>(...)",
    "C5b": "void fk::ew_vec_kernel<fk::IoBF16, 128, 1, true, false, fk::GeluOp>(...)",
    "layernorm_gelu": "void fk::layernorm_reg_kernel<fk::IoBF16, 4, 2, true, true, true, 2>(...)",
    "gelu_backward": "void fk::ew2_vec_kernel<fk::IoBF16, 128, true, false, fk::GeluBwdOp>(...)",
    "softmax_backward": "void fk::softmax_bwd_reg_kernel<fk::IoBF16, 2, 4, true, true, 2>(...)",
    "online_c5a": "void fk::softmax_rolling_kernel<fk::IoF32, 512, 4, 12, 4, true>(...)",
}


def _write_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        for d, name, value in rows:
            w.writerow({"Dispatch_Id": d, "Kernel_Name": name, "Counter_Name": counter,
                        "Counter_Value": value})


def test_ingest_counters_scales_by_the_calibration_copy(tmp_path, monkeypatch):
    # a part whose FETCH_SIZE reads half the true bytes and WRITE_SIZE all of
    # them (KiB): the copy of 1 GiB each way calibrates both; every kernel
    # moving exactly its algorithmic bytes must come out at ratio 1
    calib = 1 << 30
    fetch = [(1, NAMES["copy"], calib / 1024 / 2)]
    write = [(1, NAMES["copy"], calib / 1024)]
    d = 2
    for _ in range(2):
        for name in bench.STEP:
            half = wl.algorithmic_bytes(name) / 2  # one read and one write of equal size
            fetch.append((d, NAMES[name], half / 1024 / 2))
            write.append((d, NAMES[name], half / 1024))
            d += 1
    # the next-row kernels: reads of every input, one write (LayerNorm: x and
    # gamma/beta read, y written)
    for _ in range(2):
        for name in bench.EXTRA:
            total = bench.EXTRA_BYTES[name]
            written = 2 * 32768 * 4096 if name != "gelu_backward" else 2 * (1 << 30)
            if name == "layernorm_gelu":
                written = 32768 * 4096 * 2
            if name == "online_c5a":
                written = 1024 * 131072 * 4
            fetch.append((d, NAMES[name], (total - written) / 1024 / 2))
            write.append((d, NAMES[name], written / 1024))
            d += 1
    # a counter split over two rows of one dispatch (several agents/XCDs) is summed
    fetch[1] = (fetch[1][0], fetch[1][1], fetch[1][2] / 2)
    fetch.insert(2, fetch[1])
    _write_csv(tmp_path / "f.csv", "FETCH_SIZE", fetch)
    _write_csv(tmp_path / "w.csv", "WRITE_SIZE", write)
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", out)
    assert bench.ingest_counters(str(tmp_path / "f.csv"), str(tmp_path / "w.csv")) == 0
    rec = json.loads(out.read_text())
    assert rec["calibration"]["fetch_scale"] == pytest.approx(2.0)
    assert rec["calibration"]["write_scale"] == pytest.approx(1.0)
    for name in bench.STEP:
        k = rec["kernels"][name]
        assert k["bytes_per_launch"] == wl.algorithmic_bytes(name)
        assert k["ratio_to_algorithmic"] == 1.0
        assert k["dispatches"] == 2
    for name in bench.EXTRA:
        k = rec["next_rows"][name]
        assert k["bytes_per_launch"] == bench.EXTRA_BYTES[name]
        assert k["ratio_to_algorithmic"] == 1.0
        assert k["dispatches"] == 2
    # the figure is used only while the kernel sources hash the same
    assert bench.traffic_bytes("C5b") == wl.algorithmic_bytes("C5b")
    rec["source_hash"] = "0" * 16
    out.write_text(json.dumps(rec))
    assert bench.traffic_bytes("C5b") is None


def test_ingest_counters_refuses_swapped_files(tmp_path, monkeypatch):
    _write_csv(tmp_path / "f.csv", "FETCH_SIZE", [(1, NAMES["copy"], 1.0)])
    _write_csv(tmp_path / "w.csv", "WRITE_SIZE", [(1, NAMES["copy"], 1.0)])
    monkeypatch.setattr(bench, "TRAFFIC_FILE", tmp_path / "traffic.json")
    with pytest.raises(SystemExit):
        bench.ingest_counters(str(tmp_path / "w.csv"), str(tmp_path / "f.csv"))
    assert not (tmp_path / "traffic.json").exists()
