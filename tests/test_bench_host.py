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
    rec = {"k": {"source": "k.hip", "workload": "w1",
                 "source_sha256": hashlib.sha256(b"kernel v1\n").hexdigest(),
                 "fetch_kib_per_launch": 100.0, "fetch_scale": 2.0,
                 "write_kib_per_launch": 10.0, "write_scale": 1.0}}
    (tmp_path / "profiles" / "traffic.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "__file__", str(tmp_path / "bench.py"))
    assert bench.measured_traffic("k") == (100.0 * 2.0 + 10.0) * 1024.0
    assert bench.measured_traffic("k", "w1") == (100.0 * 2.0 + 10.0) * 1024.0
    assert bench.measured_traffic("other") is None
    # counters taken on another workload say nothing about this one
    assert bench.measured_traffic("k", "w2") is None
    src.write_text("kernel v2\n")  # the kernel changed since the counters were taken
    assert bench.measured_traffic("k") is None



def test_kernel_stats_merge_template_variants_under_the_base_name():
    recs = [("sparse_attend_kernel<true>", 0.010), ("merge_kernel", 0.002),
            ("sparse_attend_kernel<true>", 0.012), ("merge_kernel", 0.004)]
    st = bench.kernel_stats(recs, 2)
    assert set(st) == {"sparse_attend_kernel", "merge_kernel"}
    assert st["sparse_attend_kernel"]["avg_us"] == pytest.approx(11.0)
    assert st["sparse_attend_kernel"]["variants"] == ["sparse_attend_kernel<true>"]
    assert "variants" not in st["merge_kernel"]


def test_roofline_of_recorded_template_names():
    # attention dominant: the roofline must come out, keyed by the base name
    recs = [("score_table_kernel", 0.010), ("sparse_attend_kernel<true>", 0.020)]
    st = bench.kernel_stats(recs, 1)
    algo = {"score_table_kernel": ("hbm", 80e6, "x"), "sparse_attend_kernel": ("hbm", 100e6, "y")}
    r = bench.roofline_of(st, algo)
    assert r["kernel"] == "sparse_attend_kernel"
    assert r["achieved"] == pytest.approx(100e6 / 20e-6 / 1e9)
    assert r["frac"] == pytest.approx(r["achieved"] / bench.HBM_PEAK_GBS)
    # no counter record for this workload: no traffic and no rate from it
    assert bench.roofline_of(st, algo, "no-such-workload")["traffic"] is None
    assert "traffic_gbs" not in bench.roofline_of(st, algo, "no-such-workload")


def test_prefill_record_emits_attention_and_indexer_fractions():
    import numpy as np

    class Wl:
        name, batch, n_query, q_heads, kv_heads = "p", 1, 16384, 32, 4
        lens = np.array([1 << 20], np.int32)

    st = bench.kernel_stats([("score_stream_kernel", 2.0), ("select_kernel<true>", 0.3),
                             ("sparse_attend_kernel<true>", 8.0)], 1)
    rec = bench.prefill_record(Wl, [10.3], st, np)
    assert rec["indexer_mfma"]["frac"] > 0
    assert rec["attention_mfma"]["frac"] > 0
    assert rec["attention_mfma"]["unique_kv_hbm_frac"] > 0


def test_decode_algorithmic_bytes_count_the_union_of_gathered_tokens():
    import numpy as np

    class Wl:
        batch, n_query, q_heads, kv_heads = 1, 2, 8, 1
        lens = np.array([4 * 600 + 2], np.int32)   # t = 2400, 2401 share block 600

    sel = np.full((1, 2, 512), -1, np.int32)
    n_sel = np.array([[512, 512]], np.int32)
    sel[0, 0] = np.arange(512)
    sel[0, 1] = np.arange(1, 513)                  # overlaps the first row in 511 blocks
    kcmp, attn, qidx = bench.decode_bytes(Wl, sel, n_sel, np)
    assert kcmp == (2401 // 4) * 128
    union = 4 * 513 + 2                             # blocks 0..512 + tokens 2400, 2401
    assert attn == union * 1 * 128 * 2 * 2 + 2 * (2 * 8 * 128 * 2)
    assert qidx == 2 * 4 * 64 * 2
