"""bench.py end to end on the GPU: one short run of the default command prints
exactly one JSON line with the contract's fields (metric, value, unit, n_gpus,
steps, warmup, ms_per_step, higher_is_better, scaling, vs_baseline, dtype,
data, config.workload), a roofline object for the timed kernel, the FP8 leg
and the CPU oracle baseline."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_prints_one_contract_line():
    print("[case] bench.py --steps 2 --warmup 1 --cpu-budget 0.5", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "2", "--warmup", "1",
                        "--cpu-budget", "0.5"], capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout
    out = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline", "fp8"):
        assert key in out, key
    assert out["n_gpus"] == 1 and out["steps"] == 2 and out["warmup"] == 1
    assert out["unit"] == "TFLOP/s" and out["higher_is_better"] is True and out["dtype"] == "bf16"
    assert out["config"]["workload"] == "bf16_dit_b1_h56_n30272_d128"
    assert out["value"] > 0 and out["ms_per_step"] > 0
    # value is the FLOP count over the timed region
    flops = 4.0 * 56 * 30272 ** 2 * 128
    assert out["value"] == pytest.approx(flops / (out["ms_per_step"] * 1e-3) / 1e12, rel=1e-3)
    # the reported time is the median of flushed per-launch times
    t = out["timing"]
    assert "median" in t["statistic"] and t["min_ms"] <= t["median_ms"] <= t["max_ms"]
    assert out["ms_per_step"] == pytest.approx(t["median_ms"], rel=1e-3)
    roof = out["roofline"]
    assert roof["bound"] == "mfma" and roof["unit"] == "TFLOP/s" and roof["peak"] == 2500.0
    assert roof["frac"] == pytest.approx(roof["achieved"] / roof["peak"], abs=1e-4)
    assert 0 < roof["frac"] < 1
    assert roof["traffic"] is None or roof["traffic"] >= 1.7e9   # at least the algorithmic bytes
    fp8 = out["fp8"]
    assert fp8["roofline"]["peak"] == 5000.0 and 0 < fp8["roofline"]["frac"] < 1
    # counter-derived fields: null, or L2-miss (fabric) GB/s under the 8 TB/s peak and an
    # MFMA busy fraction with a plausible shader clock
    for r in (roof, fp8["roofline"]):
        assert r["fabric_gbps"] is None or 0 < r["fabric_gbps"] < 8000
        assert (r["fabric_gbps"] is None) == (r["traffic"] is None)
        assert r["mfma_busy_frac"] is None or 0 < r["mfma_busy_frac"] <= 1
        assert r["shader_clock_ghz"] is None or 0.5 < r["shader_clock_ghz"] < 3.0
    cpu = out["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["cores"] >= 1 and cpu["value"] > 0
