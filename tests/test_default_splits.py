"""The split-KV default (fa_api::default_splits, the rule behind
fa_splitkv_default_splits), on the host: its choice on the shapes it was
measured on (one MI355X, 256 CUs, DiT-style N(0,1) inputs, 1500-3000 timed
launches per point) and its invariants over a grid of shapes.

Measured TFLOP/s per number of chunks (best marked *):
  bf16 d128  8 x 4096:  1 673 | 2 751* | 3 738 | 4 683
  bf16 d128  4 x 8192:  1 713 | 2 865* | 3 865*
  bf16 d128  2 x 16384: 1 748 | 2 944  | 3 961*
  bf16 d128 16 x 2048:  1 617* | 2 595 | 3 567
  bf16 d128 32 x 1024:  1 532* | 2 427 | 3 396
  bf16 d128 12 x 4096:  1 773 | 2 819* | 3 726
  bf16 d128  8 x 8192:  1 985* | 2 915
  bf16 d128  4 x 4096:  2 524 | 3 547 | 4 606* | 6 559
  bf16 d128 20 x 4096:  1 888* | 2 853
  bf16 d128 causal 8 x 4096:  2 409 | 3 489* | 4 391
  bf16 d128 causal 16 x 4096: 1 619* | 2 553 | 3 595
  fp8  d128 32 x 1024:  1 772* | 2 482 | 3 470
  fp8  d128  4 x 4096:  3 718 | 4 776* | 6 744
  bf16 d64  causal 8 x 4096:  2 298 | 3 370* | 4 279
With the wide tiles (two waves per SIMD) on grids of at most two workgroups
per CU, re-measured (medians of 100 launches, L2 flushed):
  bf16 d128  8 x 4096:  1 682 | 2 743* | 3 694 | 4 655
  bf16 d128 causal 8 x 4096: 1 361 | 2 425 | 3 449* | 4 371
  bf16 d128  4 x 8192:  1 745 | 2 860* | 3 820
  bf16 d128  2 x 16384: 1 818 | 2 941* | 3 914
  fp8  d128  8 x 4096:  1 1142* | 2 1084 | 3 1029
  fp8  d128  4 x 8192:  1 1318 | 2 1392* | 3 1308
  fp8  d128  2 x 16384: 1 1429 | 2 1588* | 3 1533
  fp8  d128 causal 8 x 4096: 1 592 | 2 579 | 3 619*
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GXX = shutil.which("g++")

# (workgroups = B*H*ceil(N/128), N, causal) -> chunks the rule picks with 256 CUs
MEASURED = {
    (256, 4096, 0): 2, (256, 8192, 0): 2, (256, 16384, 0): 2, (256, 2048, 0): 1, (256, 1024, 0): 1,
    (384, 4096, 0): 2, (512, 8192, 0): 1, (128, 4096, 0): 4, (640, 4096, 0): 1,
    (256, 4096, 1): 3, (512, 4096, 1): 1, (256, 16384, 1): 3,
}


@pytest.fixture(scope="module")
def rule(tmp_path_factory):
    if GXX is None:
        pytest.skip("g++ not installed")
    exe = str(tmp_path_factory.mktemp("splits") / "default_splits_check")
    r = subprocess.run([GXX, "-O1", "-std=c++17", "-I" + os.path.join(ROOT, "tiled_attention_fa2_amd", "csrc"),
                        os.path.join(ROOT, "tests", "hip", "default_splits_check.cpp"), "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]

    def run(cases, which=0):
        inp = "".join(f"{c_[0]} {c_[1]} {c_[2]} {c_[3]} {c_[4] if len(c_) > 4 else 0}\n" for c_ in cases)
        out = subprocess.run([exe], input=inp, capture_output=True, text=True, timeout=60)
        assert out.returncode == 0
        return [int(line.split()[which]) for line in out.stdout.splitlines()]
    return run


# FP8 (w, N, causal) -> chunks: a non-causal grid one deep keeps chunks of
# >= 4096 keys
MEASURED_FP8 = {(256, 4096, 0): 1, (256, 8192, 0): 2, (256, 16384, 0): 2, (256, 4096, 1): 3, (512, 1024, 0): 1}


def test_choice_on_the_measured_shapes(rule):
    keys = list(MEASURED)
    got = rule([(w, n, c, 256) for w, n, c in keys])
    assert dict(zip(keys, got)) == MEASURED
    keys = list(MEASURED_FP8)
    got = rule([(w, n, c, 256, 1) for w, n, c in keys])
    assert dict(zip(keys, got)) == MEASURED_FP8


def test_invariants(rule):
    cases = [(w, n, c, cus, f) for w in (1, 7, 64, 128, 255, 256, 300, 511, 512, 513, 5000)
             for n in (1, 100, 1023, 1024, 2047, 4096, 30272, 1 << 20) for c in (0, 1) for cus in (80, 256, 304)
             for f in (0, 1)]
    for (w, n, c, cus, f), s in zip(cases, rule(cases)):
        assert 1 <= s <= 16
        if w >= 2 * cus:
            assert s == 1                          # the device is already full
        if s > 1:
            assert n // s >= 1024                  # no chunk under 1024 keys
            if not c and w >= cus:
                # nor under 2048 (bf16) / 4096 (FP8) on a grid already one deep
                assert n // s >= (4096 if f else 2048)
            # the fewest chunks that reach two (three if causal) workgroups per CU
            assert (s - 1) * w < (3 if c else 2) * cus
    # degenerate arguments
    assert rule([(0, 4096, 0, 256), (256, 0, 0, 256), (256, 4096, 0, 0)]) == [1, 1, 1]


def test_backward_dq_split_rule(rule):
    # the dQ pass (two waves per SIMD): 8 heads x 4096 tokens is 256 workgroups,
    # one per CU of a 256-CU device, so two chunks of 2048 keys
    dq = lambda cases: rule(cases, which=1)
    assert dq([(256, 4096, 0, 256), (2048, 2048, 1, 256), (13272, 30272, 0, 256)]) == [2, 1, 1]
    cases = [(w, n, c, cus) for w in (1, 7, 64, 128, 255, 256, 300, 511, 512, 513, 5000)
             for n in (1, 100, 1023, 1024, 2047, 4096, 30272, 1 << 20) for c in (0, 1) for cus in (80, 256, 304)]
    for (w, n, c, cus), s in zip(cases, dq(cases)):
        assert 1 <= s <= 8
        if w >= 2 * cus:
            assert s == 1                      # already two workgroups per CU
        if s > 1:
            assert n // s >= 1024              # no chunk under 1024 keys
            assert (s - 1) * w < 2 * cus       # the fewest chunks that reach two per CU
    assert dq([(0, 4096, 0, 256), (256, 0, 0, 256), (256, 4096, 0, 0)]) == [1, 1, 1]
