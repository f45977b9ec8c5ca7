"""bench.py's host logic without a GPU: the multi-GPU refusal, the
rocprofv3 CSV summaries (kernel statistics, calibrated traffic records,
per-kernel traffic, the shape sweep table) on small synthetic CSV files,
and the rule that a traffic record counts only for the sources it was taken
on."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

ASSIGN = "_ZN2fk12_GLOBAL__N_110k_assign16IDF16_Li4ELi4ELb1ELb1ELb0ELi4EEEvPKT_S4_PKfPiPfllli"
SUMS = "_ZN2fk12_GLOBAL__N_114k_segment_sumsIDF16_Li2ELi2ELb1EEEvPKT_PKiS6_S6_NS0_6SegOutIS2_EEllill"
COPY = ("void at::native::vectorized_elementwise_kernel<4, at::native::BinaryFunctor<float, float, "
        "float, at::native::binary_internal::MulFunctor<float> >, std::array<char*, 3ul> >(int, "
        "at::native::BinaryFunctor<float, float, float, at::native::binary_internal::MulFunctor<float> "
        ">, std::array<char*, 3ul>)")


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = run_bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def write_counters(path, counter, rows):
    """rows: (kernel name, value in KiB) per dispatch."""
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, v in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": v})


def test_stats_summary(tmp_path):
    p = tmp_path / "stats.csv"
    with open(p, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Name", "Calls", "TotalDurationNs", "AverageNs",
                                          "Percentage", "MinNs", "MaxNs", "StdDev"])
        w.writeheader()
        w.writerow({"Name": ASSIGN, "Calls": 13, "TotalDurationNs": 6500000,
                    "AverageNs": 500000.0, "Percentage": 80.0, "MinNs": 490000,
                    "MaxNs": 510000, "StdDev": 1.0})
    r = run_bench("--summarize", "stats", str(p), "the", "command")
    assert r.returncode == 0, r.stderr
    assert "command: `the command`" in r.stdout
    assert "| k_assign16 | 13 | 500.0 | 490.0 | 510.0 | 80.00 |" in r.stdout


def test_traffic_record_is_calibrated_by_the_copy(tmp_path):
    # the copy kernel's counter reads half the true 1 GiB for FETCH_SIZE and
    # all of it for WRITE_SIZE: the assign's figures are scaled the same way
    f, w = tmp_path / "fetch.csv", tmp_path / "write.csv"
    write_counters(f, "FETCH_SIZE", [(ASSIGN, 1000.0), (ASSIGN, 1200.0), (COPY, 524288.0),
                                     (COPY, 10.0)])
    write_counters(w, "WRITE_SIZE", [(ASSIGN, 50.0), (ASSIGN, 50.0), (COPY, 1048576.0)])
    r = run_bench("--summarize", "traffic", str(f), str(w), "wl", "cmd")
    assert r.returncode == 0, r.stderr
    rec = json.loads(r.stdout)
    assert rec["counters"]["FETCH_SIZE"]["calibration_factor"] == pytest.approx(2.0)
    assert rec["counters"]["WRITE_SIZE"]["calibration_factor"] == pytest.approx(1.0)
    assert rec["hbm_bytes_per_launch"] == round((1100.0 * 2.0 + 50.0) * 1024)
    assert rec["assign_sources_sha256_16"] == bench.assign_sources_hash()


def test_traffic_kernels_record(tmp_path):
    f, w = tmp_path / "fetch.csv", tmp_path / "write.csv"
    write_counters(f, "FETCH_SIZE", [(SUMS, 100.0), (SUMS, 300.0), (COPY, 524288.0)])
    write_counters(w, "WRITE_SIZE", [(SUMS, 10.0), (SUMS, 10.0), (COPY, 1048576.0)])
    r = run_bench("--summarize", "traffic-kernels", str(f), str(w), "wl", "cmd")
    assert r.returncode == 0, r.stderr
    rec = json.loads(r.stdout)["kernels"]["k_segment_sums"]
    assert rec["dispatches"] == 2
    assert rec["FETCH_SIZE_MB_per_dispatch"] == pytest.approx(200.0 * 1024 * 2.0 / 1e6, abs=1e-3)
    assert rec["WRITE_SIZE_MB_per_dispatch"] == pytest.approx(10.0 * 1024 / 1e6, abs=1e-3)


def test_sweep_table_marks_the_library_shape(tmp_path):
    rows = [{"d": 64, "point_blocks": nb, "waves": w, "grid_wgs": 0, "ms": ms, "TFLOPs": 1.0,
             "labels_identical": True}
            for nb, w, ms in ((4, 4, 0.30), (8, 4, 0.32))]
    rec = {"rows": rows, "per_d": [{"d": 64, "library_shape": {"point_blocks": 4, "waves": 4},
                                    "library_choice_ms": 0.30, "best": rows[0],
                                    "library_loss_pct": 0.0}]}
    p = tmp_path / "sweep.json"
    p.write_text(json.dumps(rec) + "\n")
    r = run_bench("--summarize", "sweep", str(p), "cmd")
    assert r.returncode == 0, r.stderr
    assert "| 4 | 4 | one per block (library) | 0.3 |" in r.stdout
    assert "| 8 | 4 | one per block | 0.32 |" in r.stdout
    assert "library loss 0.0 %" in r.stdout


def test_traffic_counts_only_for_the_sources_it_was_taken_on(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    rec = {"hbm_bytes_per_launch": 123, "assign_sources_sha256_16": "abc"}
    (tmp_path / "profiles" / "traffic_assign_wl.json").write_text(json.dumps(rec))
    assert bench.measured_traffic("wl", "abc") == 123
    assert bench.measured_traffic("wl", "other") is None
    assert bench.measured_traffic("missing", "abc") is None


def test_unknown_summary_kind():
    r = run_bench("--summarize", "nonsense")
    assert r.returncode == 2


def test_input_hash_is_the_sha256_of_the_bytes():
    import hashlib

    import numpy as np
    import torch
    x = torch.tensor([[1.0, -2.5], [0.25, 3.0]], dtype=torch.float16)
    raw = np.array([0x3C00, 0xC100, 0x3400, 0x4200], dtype="<u2").tobytes()
    assert bench.tensor_sha256_16(x) == hashlib.sha256(raw).hexdigest()[:16]
    y = torch.tensor([1.0, 2.0], dtype=torch.float32)
    assert bench.tensor_sha256_16(y) == hashlib.sha256(np.array([1.0, 2.0], "<f4").tobytes()).hexdigest()[:16]
