"""Builds libfa.so (the HIP kernels and the C ABI of include/fa.h) in-tree for
gfx950 with hipcc. Run as `python -m tiled_attention_fa2_amd.build`."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libfa.so")
SOURCES = [os.path.join(PKG, "csrc", f) for f in ("fa_api.hip", "fa_quant_api.hip", "fa_bwd_api.hip")]
HEADERS = [os.path.join(ROOT, "include", "fa.h"),
           os.path.join(PKG, "csrc", "fa_api_common.hpp"),
           os.path.join(PKG, "csrc", "fa_bwd_kernel.hpp"),
           os.path.join(PKG, "csrc", "fa_fwd_kernel.hpp"),
           os.path.join(PKG, "csrc", "fa_merge_kernel.hpp"),
           os.path.join(PKG, "csrc", "fa_quant_kernel.hpp")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 VALU forms stay off: ordinary float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(PKG, "csrc"),
]


PROBE_SRC = os.path.join(ROOT, "tests", "hip", "mfma_probe.hip")
PROBE_LIB = os.path.join(ROOT, "tests", "hip", "libmfma_probe.so")
VARIANTS_SRC = os.path.join(ROOT, "tests", "hip", "stage_variants.hip")
VARIANTS_LIB = os.path.join(ROOT, "tests", "hip", "libstage_variants.so")


def _hipcc(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed: " + " ".join(cmd[-3:]))


def build_probe(verbose: bool = False) -> str:
    """The test helpers of tests/hip: the one-wave MFMA layout/precision probe
    and the forward kernel at other pipeline depths (the determinism test),
    both used by the GPU tests."""
    _hipcc([HIPCC, *FLAGS, PROBE_SRC, "-o", PROBE_LIB + ".tmp"], verbose)
    os.replace(PROBE_LIB + ".tmp", PROBE_LIB)
    if os.path.exists(VARIANTS_SRC):
        _hipcc([HIPCC, *FLAGS, VARIANTS_SRC, "-o", VARIANTS_LIB + ".tmp"], verbose)
        os.replace(VARIANTS_LIB + ".tmp", VARIANTS_LIB)
    return PROBE_LIB


def build(verbose: bool = False, extra=()) -> str:
    _hipcc([HIPCC, *FLAGS, *extra, *SOURCES, "-o", LIB + ".tmp"], verbose)
    os.replace(LIB + ".tmp", LIB)
    if os.path.exists(PROBE_SRC):
        build_probe(verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
