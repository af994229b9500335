"""bench.py's host-side logic (no GPU): the one-GPU guard, per-kernel
aggregation of the timing records, and the counter-based traffic record that
is dropped once the kernel's source changes."""
import hashlib
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_kernel_stats_averages_per_name():
    recs = [("a", 1.0), ("b", 2.0), ("a", 3.0), ("b", 4.0)]
    st = bench.kernel_stats(recs, 2)
    assert st["a"] == {"avg_us": 2000.0, "launches_per_step": 1.0}
    assert st["b"] == {"avg_us": 3000.0, "launches_per_step": 1.0}


def test_traffic_record_follows_the_source(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("kernel v1\n")
    (tmp_path / "profiles").mkdir()
    rec = {"k": {"source": "k.hip",
                 "source_sha256": hashlib.sha256(b"kernel v1\n").hexdigest(),
                 "fetch_kib_per_launch": 100.0, "fetch_scale": 2.0,
                 "write_kib_per_launch": 10.0, "write_scale": 1.0}}
    (tmp_path / "profiles" / "traffic.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "__file__", str(tmp_path / "bench.py"))
    assert bench.measured_traffic("k") == (100.0 * 2.0 + 10.0) * 1024.0
    assert bench.measured_traffic("other") is None
    src.write_text("kernel v2\n")  # the kernel changed since the counters were taken
    assert bench.measured_traffic("k") is None

