"""Host logic of bench.py, on the CPU: the one-GPU refusal, the kernel-source
hash that decides whether the committed HBM-traffic counters still describe
the kernel, and the CPU baseline leg (the oracle on a bounded sample)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from tiled_attention_fa2_amd.inputs import WORKLOADS, make_qkv  # noqa: E402


def test_more_than_one_gpu_is_refused_before_any_device_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""          # no JSON line


def test_source_hash_ignores_comments_and_spacing(tmp_path, monkeypatch):
    a = tmp_path / "k.hpp"
    a.write_text("// the kernel\nint f(int x) {\n  return x + 1;   /* one */\n}\n")
    monkeypatch.setattr(bench, "KERNEL_SOURCES", [str(a)])
    h0 = bench.kernel_source_hash()
    a.write_text("// reworded comment\n\nint f(int x)   {\n    return x + 1;  /* a longer\n comment */\n}\n")
    assert bench.kernel_source_hash() == h0
    a.write_text("// the kernel\nint f(int x) {\n  return x + 2;   /* one */\n}\n")
    assert bench.kernel_source_hash() != h0


def test_traffic_is_reported_only_for_the_source_it_was_taken_on(monkeypatch):
    name = "bf16_dit_b1_h56_n30272_d128"
    with open(os.path.join(ROOT, "profiles", f"fa_fwd_{name}_traffic.json")) as f:
        rec = json.load(f)
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: rec["source_sha256"])
    t = bench.measured_traffic(name)
    assert t == rec["fabric_bytes_per_launch"]
    # read + write, each a counter scaled by the copy calibration
    assert t == rec["fabric_read_bytes"] + rec["fabric_write_bytes"]
    assert rec["fabric_read_bytes"] == pytest.approx(rec["fetch_size_kib"] * 1024 * rec["fetch_scale"], rel=1e-6)
    assert rec["fabric_write_bytes"] == pytest.approx(rec["write_size_kib"] * 1024 * rec["write_scale"], rel=1e-6)
    # HBM traffic can not be below the algorithmic bytes (Q, K, V read, O, L written once)
    assert t >= rec["algorithmic_bytes"]
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 64)
    assert bench.measured_traffic(name) is None
    assert bench.measured_traffic("no_such_workload") is None


def test_flop_accounting():
    w = WORKLOADS["bf16_dit_b1_h56_n30272_d128"]
    assert w.flops() == 4.0 * 1 * 56 * 30272 ** 2 * 128
    c = WORKLOADS["bf16_causal_b4_h32_n2048_d128"]
    assert c.flops() == 0.5 * 4.0 * 4 * 32 * 2048 ** 2 * 128


def test_cpu_baseline_leg_times_the_oracle_on_a_sample():
    w = WORKLOADS["f32_b1_h1_n256_d64"]
    q, k, v = make_qkv(w.B, w.H, w.N, w.d, "f32", seed=0)
    out = bench.cpu_baseline(w, q, k, v, budget_s=0.2)
    assert out["kind"] == "oracle" and out["unit"] == "TFLOP/s"
    assert out["value"] > 0 and out["cores"] >= 1
    assert "query rows" in out["sample"] and w.name in out["sample"]
    assert out["extrapolated_full_problem_s"] > 0


def test_counter_fields_follow_the_source_they_were_taken_on(monkeypatch, tmp_path):
    rec = {"source_sha256": "a" * 64, "workloads": {"bf16_dit_b1_h56_n30272_d128": {
        "kernel": "k", "mfma_busy_frac": 0.63, "shader_clock_ghz": 1.67, "duration_ms": 23.9}}}
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "fa_fwd_dit_mfma_utilisation.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "a" * 64)
    f = bench.counter_fields("bf16_dit_b1_h56_n30272_d128", 8.0e9, 25.0)
    assert f == {"fabric_gbps": 320.0, "mfma_busy_frac": 0.63, "shader_clock_ghz": 1.67}
    # no traffic record: no bandwidth; a split run: nothing (the counters are of the unsplit kernel)
    assert bench.counter_fields("bf16_dit_b1_h56_n30272_d128", None, 25.0)["fabric_gbps"] is None
    assert set(bench.counter_fields("bf16_dit_b1_h56_n30272_d128", 8.0e9, 25.0, False).values()) == {None}
    assert bench.counter_fields("no_such_workload", None, 1.0)["mfma_busy_frac"] is None
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "b" * 64)
    assert bench.counter_fields("bf16_dit_b1_h56_n30272_d128", 8.0e9, 25.0)["mfma_busy_frac"] is None


def test_timing_statistic_is_the_median():
    # the reported time is the median of the per-launch times, as the pages'
    # harness reports; mean, min and max ride along
    import bench

    st = bench.stats([3.0, 1.0, 2.0])
    assert st == {"median_ms": 2.0, "mean_ms": 2.0, "min_ms": 1.0, "max_ms": 3.0}
    assert bench.stats([4.0, 1.0, 2.0, 3.0])["median_ms"] == 2.5
    assert bench.stats([5.0, 1.0, 1.0, 1.0, 9.0])["median_ms"] == 1.0
    assert bench.FLUSH_BYTES >= 512 << 20
