"""The kernels' block -> work-item map, checked on the host: tests/hip/
work_item_check.cpp compiles the real header (host code only) and checks, for
2520 shapes (heads, query tiles, key splits, no / head-by-head / across-heads
causal order), that every block index lands on a distinct (head, tile) item
and every item is covered, that both causal orders hand each head's tiles
on one XCD out longest first, and that the across-heads order with whole
heads per XCD hands each XCD's slots out longest query tile first."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None, reason="hipcc not installed")
def test_work_item_map_is_a_bijection_and_causal_longest_first(tmp_path):
    exe = str(tmp_path / "work_item_check")
    cmd = [HIPCC, "-x", "hip", "--cuda-host-only", "-O1", "-std=c++17",
           "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(ROOT, "tiled_attention_fa2_amd", "csrc"),
           os.path.join(ROOT, "tests", "hip", "work_item_check.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr
