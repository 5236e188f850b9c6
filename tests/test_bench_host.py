"""Host logic of bench.py, on the CPU: the refusal of more than one GPU, the
staleness check of the committed traffic summary (its figure is used only
while the split kernel's source matches the hash it records), and the
scaling of FETCH_SIZE / WRITE_SIZE counts by a plain copy's counts."""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stdout


def test_traffic_summary_matches_the_kernel_source():
    """The committed summary was taken on the current split kernel, and its
    read traffic is within a few percent of the algorithmic bytes."""
    lat = 16 * 2048 * (32 * 64 + 512) * 2
    t = bench.read_traffic(lat)
    assert t is not None
    assert 1.0 <= t / lat < 1.1


def test_traffic_summary_goes_stale_when_the_kernel_changes(monkeypatch):
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0000000000000000")
    assert bench.read_traffic(1) is None


def _write_rows(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_counter_scaling_by_the_copy(tmp_path):
    """Counts of the split kernel are scaled by the bytes per counted unit
    that the 256 MiB copies show (small copies are ignored)."""
    copy_units_f, copy_units_w = 131072.0, 262144.0   # 2048 and 1024 bytes per unit
    split_f, split_w = 81920.0, 8704.0
    fetch = tmp_path / "fetch.csv"
    write = tmp_path / "write.csv"
    _write_rows(fetch, "FETCH_SIZE", [("__amd_rocclr_copyBuffer", 3.0),
                                      ("__amd_rocclr_copyBuffer", copy_units_f),
                                      ("decode_split_kernel<...>", split_f),
                                      ("decode_split_kernel<...>", split_f),
                                      ("finish_kernel<...>", 99.0)])
    _write_rows(write, "WRITE_SIZE", [("__amd_rocclr_copyBuffer", copy_units_w),
                                      ("decode_split_kernel<...>", split_w)])
    out = tmp_path / "summary.txt"
    bench.summarize_pmc(str(fetch), str(write), str(out))
    kv = dict(line.strip().split("=", 1) for line in open(out)
              if "=" in line and not line.startswith("#"))
    assert float(kv["fetch_bytes_per_unit"]) == pytest.approx(2048.0)
    assert float(kv["write_bytes_per_unit"]) == pytest.approx(1024.0)
    assert float(kv["hbm_read_bytes_per_launch"]) == pytest.approx(split_f * 2048.0, rel=1e-6)
    assert float(kv["hbm_write_bytes_per_launch"]) == pytest.approx(split_w * 1024.0, rel=1e-6)
    assert int(kv["dispatches_fetch"]) == 2
    assert kv["kernel_source_sha"] == bench.kernel_source_hash()
