"""Issue cost of the softmax's VALU operations on one MI355X SIMD
(tests/hip/valu_rates.hip), the measurement behind not emulating exp2 on FMA
units ("Kernels and Memory in LLM Inference", section "FlashAttention-4": part
of the exponentials computed by polynomial on FMA units while the special-
function unit does the rest). Two waves share each SIMD; the test prints the
time of each pairing and checks only what the design relies on: an FMA
polynomial exp2 costs more than v_exp_f32, and v_exp_f32 next to an FMA wave
does not run as if on a separate unit (the pair takes clearly longer than
the exp wave alone). Each time is the fastest of three launches.
"""
import ctypes
import os

import pytest
import torch

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(__file__), "hip", "libvalu_rates.so")


def test_valu_issue_costs():
    assert torch.cuda.is_available()
    lib = ctypes.CDLL(LIB)
    lib.valu_pair_run.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_float)]
    lib.poly_exp2_error.argtypes = [ctypes.POINTER(ctypes.c_float)]
    t = {}
    for pair, name in ((10, "fma"), (20, "exp"), (30, "poly exp2"), (11, "fma+fma"), (22, "exp+exp"),
                       (12, "fma+exp"), (23, "exp+poly")):
        runs = []
        for _ in range(3):          # the fastest of three: noise only slows a run
            us = ctypes.c_float(0.0)
            assert lib.valu_pair_run(pair, 1000, ctypes.byref(us)) == 0
            runs.append(us.value)
        t[name] = min(runs)
    err = ctypes.c_float(0.0)
    assert lib.poly_exp2_error(ctypes.byref(err)) == 0
    print("us per launch: " + ", ".join(f"{k} {v:.0f}" for k, v in t.items()), flush=True)
    print(f"FMA exp2 max relative error vs v_exp_f32 on [-30, 0]: {err.value:.2e}", flush=True)
    assert t["poly exp2"] > t["exp"]
    assert t["fma+exp"] > 1.15 * t["exp"]
    assert err.value < 1e-4
