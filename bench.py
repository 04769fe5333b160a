"""Benchmark of the FlashAttention-2 forward on one MI355X.

Default workload: the MiniMax H3 DiT self-attention shape the pages measure
("1.8x Faster Attention on an RTX 5080", section "The attention itself"):
B=1, H=56, N=30272, d=128, non-causal, bf16, with iid N(0,1) synthetic inputs
in place of the model's activations. The same shape in FP8-e4m3 (per-head
quantised from the same bf16 draws) is timed next to it.

A step is one fa_fwd over the whole batch with inputs resident in HBM; 1 GiB is
written before each timed launch (outside its event pair) so that neither L2 nor
the MALL holds them, and the reported time is the median per-launch time.
FLOP per step = 4*B*H*N^2*d (halved for causal), the pages' accounting.
Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s and % of MFMA peak (bf16 / fp8), H=56 N=30272 d=128"
PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3}   # MI355X dense MFMA
KERNEL_SOURCES = ["tiled_attention_fa2_amd/csrc/fa_fwd_kernel.hpp",
                  "tiled_attention_fa2_amd/csrc/fa_api_common.hpp",
                  "tiled_attention_fa2_amd/csrc/fa_api_device.hpp",
                  "tiled_attention_fa2_amd/csrc/fa_api.hip"]


def kernel_source_hash() -> str:
    """Hash of the forward kernel's code: the sources with comments and blank
    space removed, so that a change of wording alone keeps the recorded
    traffic counters valid."""
    import re

    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p)) as f:
            txt = f.read()
        txt = re.sub(r"/\*.*?\*/", " ", txt, flags=re.S)
        txt = re.sub(r"//[^\n]*", " ", txt)
        h.update(" ".join(txt.split()).encode())
    return h.hexdigest()


def kernel_name(w, num_splits: int = 1) -> str:
    """The kernel fa_fwd launches for this workload (bf16 and fp8 use the DMA +
    transpose-read kernel, fp32 the register-staged one); with key chunks, the
    merge follows."""
    k = "fa_fwd_dma_kernel" if w.dtype in ("bf16", "fp8") else "fa_fwd_kernel"
    return k + " + fa_merge_kernel" if num_splits > 1 else k


def measured_traffic(workload: str):
    """L2-miss (fabric) bytes per launch from the committed rocprofv3 --pmc summary, only if
    it was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"fa_fwd_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_sha256") != kernel_source_hash():
        return None
    return t.get("fabric_bytes_per_launch")


def measured_mfma(workload: str):
    """MFMA busy fraction and shader clock of the workload's kernel from the
    committed rocprofv3 --pmc record (SQ_VALU_MFMA_BUSY_CYCLES, SQ_CYCLES),
    only if it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "fa_fwd_dit_mfma_utilisation.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_sha256") != kernel_source_hash():
        return None
    return t.get("workloads", {}).get(workload)


def counter_fields(workload: str, traffic, kern_ms: float, unsplit: bool = True) -> dict:
    """The roofline object's counter-derived fields: fabric GB/s (the counted
    L2-miss bytes over the live kernel time; FETCH_SIZE and WRITE_SIZE count
    what the L2 reads from and writes to the fabric, MALL hits included, so
    this is an upper bound on HBM traffic: no HBM-only counter exists) and the MFMA busy fraction and clock. The
    counters describe the unsplit kernel: a split-KV run gets None."""
    if not unsplit:
        return {"fabric_gbps": None, "mfma_busy_frac": None, "shader_clock_ghz": None}
    m = measured_mfma(workload)
    return {"fabric_gbps": round(traffic / (kern_ms * 1e-3) / 1e9, 1) if traffic else None,
            "mfma_busy_frac": m["mfma_busy_frac"] if m else None,
            "shader_clock_ghz": m["shader_clock_ghz"] if m else None}


FLUSH_BYTES = 1 << 30    # more than the L2 (8 x 4 MiB) and the 256 MiB MALL together


def make_flush(torch, device):
    """A 1 GiB buffer; writing it before a timed launch evicts the inputs from
    L2 and MALL, as the pages' harness does ("FlashAttention-2 from PyTorch to
    Triton", the harness paragraph: do_bench flushes L2 between runs)."""
    return torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=device)


def timed_launches(torch, launch, steps, flush):
    """Time exactly `steps` launches, each alone between two HIP events on the
    current stream, with the flush buffer written before each one (outside
    the event pair). Returns the per-launch times in ms."""
    stream = torch.cuda.current_stream()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        flush.fill_(i & 0xFF)
        starts[i].record(stream)
        launch()
        ends[i].record(stream)
    torch.cuda.synchronize()
    return [s.elapsed_time(e) for s, e in zip(starts, ends)]


def stats(times):
    """Median (the reported statistic, as do_bench reports), mean, min, max."""
    t = sorted(times)
    n = len(t)
    med = t[n // 2] if n % 2 else 0.5 * (t[n // 2 - 1] + t[n // 2])
    return {"median_ms": med, "mean_ms": sum(t) / n, "min_ms": t[0], "max_ms": t[-1]}


def time_fwd(fa, torch, args_in, kw, steps, warmup, flush, fn=None):
    """Warm up, then time exactly `steps` launches of fn (default fa.fwd), the
    caches flushed before each. Returns the per-launch statistics (ms)."""
    fn = fa.fwd if fn is None else fn
    splits = kw.get("num_splits") or 1
    if splits > 1:   # the split-KV workspace, allocated once outside the timed region
        B, H, N, d = args_in[0].shape
        kw = dict(kw, workspace=torch.empty(fa.splitkv_workspace_bytes(B, H, N, d, splits),
                                            dtype=torch.uint8, device=args_in[0].device))
    o, lse = fn(*args_in, **kw)
    kw = dict(kw, out=o, lse=lse)
    for _ in range(warmup):
        fn(*args_in, **kw)
    return stats(timed_launches(torch, lambda: fn(*args_in, **kw), steps, flush))


def time_bwd(fa, torch, w, qd, kd, vd, steps, warmup, flush):
    """The backward on the workload's own inputs: fwd once for O and L, a
    seeded dO, then `steps` timed fa_bwd calls (HIP events on the stream,
    caches flushed before each); returns the median ms."""
    from tiled_attention_fa2_amd.inputs import make_dout

    o, lse = fa.fwd(qd, kd, vd, causal=w.causal, scale=w.scale, num_splits=1)
    do = make_dout(w.B, w.H, w.N, w.d, seed=1).to(qd.device)
    ws = torch.empty(fa.bwd_workspace_bytes(w.B, w.H, w.N), dtype=torch.uint8, device=qd.device)
    dq, dk, dv = fa.bwd(qd, kd, vd, o, lse, do, causal=w.causal, scale=w.scale, workspace=ws)
    kw = dict(causal=w.causal, scale=w.scale, dq=dq, dk=dk, dv=dv, workspace=ws)
    for _ in range(warmup):
        fa.bwd(qd, kd, vd, o, lse, do, **kw)
    return stats(timed_launches(torch, lambda: fa.bwd(qd, kd, vd, o, lse, do, **kw), steps, flush))["median_ms"]


def cpu_baseline(w, q, k, v, budget_s: float):
    """Time the fp64 oracle on a bounded sample of the same workload: chunks of
    128 query rows against all N keys, cycling over heads, until budget_s."""
    import numpy as np

    import oracle

    try:
        from threadpoolctl import threadpool_info

        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    qn = q.float().numpy()
    kn = k.float().numpy()
    vn = v.float().numpy()
    group = w.H // w.kv_heads          # grouped-query attention: query head h reads K/V head h // group
    rows_done = 0
    t0 = time.perf_counter()
    h = 0
    r0 = 0
    while time.perf_counter() - t0 < budget_s:
        rows = np.arange(r0, min(r0 + 128, w.N))
        hk = h // group
        oracle.attention(qn[:, h:h + 1], kn[:, hk:hk + 1], vn[:, hk:hk + 1], w.scale,
                         causal=w.causal, rows=rows)
        rows_done += len(rows)
        h = (h + 1) % w.H
        r0 = (r0 + 128) % w.N
    dt = time.perf_counter() - t0
    flops = 4.0 * w.d * w.N * rows_done      # non-causal: every row sees N keys
    if w.causal:
        flops *= 0.5                         # the pages' convention: half the pairs
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "unknown")
    except OSError:
        pass
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "cpu_model": cpu_model,
            "sample": f"{rows_done} query rows x all {w.N} keys (chunks of 128 rows, cycling heads) "
                      f"of {w.name}, fp64 numpy, {dt:.1f} s",
            "extrapolated_full_problem_s": dt * (w.B * w.H * w.N) / rows_done}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="bf16_dit_b1_h56_n30272_d128")
    ap.add_argument("--no-fp8", action="store_true", help="skip the FP8 leg")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle work for cpu_baseline (0 = skip)")
    ap.add_argument("--num-splits", type=int, default=None,
                    help="key chunks of the split-KV path (default: the library's choice; 1 = unsplit)")
    ap.add_argument("--bwd", action="store_true",
                    help="also time the backward pass (bf16 workloads) into a 'bwd' object")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB first (a kernel of known "
                         "traffic, to scale rocprofv3 FETCH_SIZE / WRITE_SIZE counters)")
    a = ap.parse_args()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {a.gpus} is not supported "
              "(the forward shards by head with no exchange; see the design notes)", file=sys.stderr)
        sys.exit(2)

    import torch

    from tiled_attention_fa2_amd import fa
    from tiled_attention_fa2_amd.inputs import WORKLOADS, make_qkv, make_signs, make_workload

    w = WORKLOADS[a.workload]
    dev = torch.device("cuda:0")
    if a.copy_probe_mib > 0:
        n = a.copy_probe_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] copy probe: {a.copy_probe_mib} MiB read + {a.copy_probe_mib} MiB written",
              file=sys.stderr, flush=True)
        del src, dst
    print(f"[bench] generating {w.name} inputs", file=sys.stderr, flush=True)
    if w.dtype == "fp8":   # fp8 workloads quantise the bf16 draws on the device
        q, k, v = make_qkv(w.B, w.H, w.N, w.d, "bf16", seed=0)
    else:
        _, (q, k, v) = make_workload(w.name, seed=0)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)

    code = {"f32": fa.DTYPE_F32, "bf16": fa.DTYPE_BF16, "fp8": fa.DTYPE_FP8_E4M3}[w.dtype]
    splits = a.num_splits if a.num_splits is not None else fa.default_splits(w.B, w.H, w.N, w.d, w.causal, code)
    if w.dtype == "fp8":
        q8, k8, v8, ds = fa.quantize_qkv_fp8(qd, kd, vd)
        main_in, main_kw = (q8, k8, v8), dict(causal=w.causal, scale=w.scale, descales=ds, num_splits=splits)
    else:
        main_in, main_kw = (qd, kd, vd), dict(causal=w.causal, scale=w.scale, num_splits=splits)
    flush = make_flush(torch, dev)
    print("[bench] timing main leg", file=sys.stderr, flush=True)
    t_main = time_fwd(fa, torch, main_in, main_kw, a.steps, a.warmup, flush)
    ms = kern_ms = t_main["median_ms"]
    flops = w.flops()
    value = flops / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    achieved = value
    traffic = measured_traffic(w.name)
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Hkv": w.kv_heads, "N": w.N, "d": w.d,
                   "causal": w.causal, "num_splits": splits,
                   "pct_of_mfma_peak": round(100 * value / peak, 2)},
        "timing": {"statistic": "median of the per-launch HIP event times; 1 GiB written before each "
                                "launch, outside the event pair, to flush L2 and MALL",
                   **{k: round(x, 4) for k, x in t_main.items()}},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": traffic if splits == 1 else None,
                     "kernel": kernel_name(w, splits), "kernel_ms": round(kern_ms, 4),
                     **counter_fields(w.name, traffic, kern_ms, splits == 1)},
    }

    if not a.no_fp8 and w.name == "bf16_dit_b1_h56_n30272_d128":
        w8 = WORKLOADS["fp8_dit_b1_h56_n30272_d128"]
        print("[bench] timing fp8 leg", file=sys.stderr, flush=True)
        q8, k8, v8, ds = fa.quantize_qkv_fp8(qd, kd, vd)
        splits8 = a.num_splits if a.num_splits is not None else fa.default_splits(
            w8.B, w8.H, w8.N, w8.d, w8.causal, fa.DTYPE_FP8_E4M3)
        t8 = time_fwd(fa, torch, (q8, k8, v8), dict(causal=False, scale=w8.scale, descales=ds, num_splits=splits8),
                      a.steps, a.warmup, flush)
        ms8 = kern8 = t8["median_ms"]
        # per-head quantise of Q, K and V (the FP8 path's first step), timed on its own
        qms = stats(timed_launches(torch, lambda: fa.quantize_qkv_fp8(qd, kd, vd), a.steps, flush))["median_ms"]
        # the same with Q and K rotated by a randomised Hadamard transform first
        signs = make_signs(w8.d, seed=0).to(dev)
        fa.quantize_qkv_fp8(qd, kd, vd, signs=signs)
        rqms = stats(timed_launches(torch, lambda: fa.quantize_qkv_fp8(qd, kd, vd, signs=signs), a.steps,
                                    flush))["median_ms"]
        # per-block FP8: row-block quantise of Q and K, key-block quantise of
        # V (one pass each), then the forward with the scales in the MFMAs
        mq8, mk8, mv8, msc = fa.quantize_qkv_mxfp8(qd, kd, vd)
        tm = time_fwd(fa, torch, (mq8, mk8, mv8, msc), dict(causal=False, scale=w8.scale, num_splits=splits8),
                      a.steps, a.warmup, flush, fn=fa.fwd_mxfp8)
        msm = mskern = tm["median_ms"]
        mqms = stats(timed_launches(torch, lambda: fa.quantize_qkv_mxfp8(qd, kd, vd), a.steps, flush))["median_ms"]
        del mq8, mk8, mv8, msc
        v8 = w8.flops() / (ms8 * 1e-3) / 1e12
        out["fp8"] = {
            "workload": w8.name, "value": round(v8, 2), "unit": "TFLOP/s", "ms_per_step": round(ms8, 4),
            "timing": {k: round(x, 4) for k, x in t8.items()},
            "pct_of_mfma_peak": round(100 * v8 / PEAK_TFLOPS["fp8"], 2),
            "quantize_qkv_ms": round(qms, 4),
            "value_incl_quantize": round(w8.flops() / ((ms8 + qms) * 1e-3) / 1e12, 2),
            "quantize_qkv_rotated_ms": round(rqms, 4),
            "value_incl_rotated_quantize": round(w8.flops() / ((ms8 + rqms) * 1e-3) / 1e12, 2),
            "per_block": {"value": round(w8.flops() / (msm * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
                          "ms_per_step": round(msm, 4), "kernel_ms": round(mskern, 4),
                          "pct_of_mfma_peak": round(100 * w8.flops() / (msm * 1e-3) / 1e12 / PEAK_TFLOPS["fp8"], 2),
                          "quantize_qkv_ms": round(mqms, 4),
                          "value_incl_quantize": round(w8.flops() / ((msm + mqms) * 1e-3) / 1e12, 2),
                          "scales": "E8M0 per 32 elements along each product's contraction axis"},
            "roofline": {"bound": "mfma", "achieved": round(w8.flops() / (kern8 * 1e-3) / 1e12, 2),
                         "peak": PEAK_TFLOPS["fp8"], "unit": "TFLOP/s",
                         "frac": round(w8.flops() / (kern8 * 1e-3) / 1e12 / PEAK_TFLOPS["fp8"], 4),
                         "traffic": measured_traffic(w8.name) if splits8 == 1 else None,
                         "kernel": kernel_name(w8, splits8),
                         "kernel_ms": round(kern8, 4),
                         **counter_fields(w8.name, measured_traffic(w8.name), kern8, splits8 == 1)},
        }

    if a.bwd and w.dtype == "bf16":
        print("[bench] timing the backward", file=sys.stderr, flush=True)
        msb = time_bwd(fa, torch, w, qd, kd, vd, a.steps, a.warmup, flush)
        fb = 2.5 * flops     # five N x N x d products against the forward's two
        out["bwd"] = {"value": round(fb / (msb * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "ms_per_step": round(msb, 4),
                      "flop_convention": "10*B*H*N^2*d (halved for causal): dV, dP, dS-to-dQ, dS-to-dK and the "
                                         "recomputed S; the kernels execute 14*B*H*N^2*d on MFMA (S and dP again "
                                         "in the dQ pass)",
                      "pct_of_mfma_peak": round(100 * fb / (msb * 1e-3) / 1e12 / peak, 2),
                      "mfma_executed_tflops": round(1.4 * fb / (msb * 1e-3) / 1e12, 2)}

    if a.cpu_budget > 0:
        print("[bench] timing the CPU oracle sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, q, k, v, a.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
