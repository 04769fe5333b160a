"""Determinism across pipeline depths: the race detector.

The forward kernel fa_fwd launches (head dim 128, bf16 and FP8) is built again
by tests/hip/stage_variants.hip with 2 and 3 LDS stages, with MFMA operand
reads 1 and 2 steps ahead, and with each tile's prefetch issued before or after
its QK MFMAs. None of these changes which values are added in which order;
they change only when K/V tiles land in LDS and when operands are read. So every variant must reproduce fa_fwd's O and L bit for bit: a missing
wait or barrier (a tile read before it landed, or overwritten while a slower
wave still reads it) would show up as a difference.
"""
import ctypes
import math
import os

import pytest
import torch

from tiled_attention_fa2_amd import fa
from tiled_attention_fa2_amd.inputs import make_qkv

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "tests", "hip", "libstage_variants.so")


def _lib():
    if not os.path.exists(LIB):
        pytest.fail("tests/hip/libstage_variants.so is not built (python -m tiled_attention_fa2_amd.build)")
    lib = ctypes.CDLL(LIB)
    lib.fa_test_fwd_variant.restype = ctypes.c_int
    lib.fa_test_fwd_variant.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 4 + [ctypes.c_float, ctypes.c_int,
                                        ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_void_p]
    return lib


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("causal", [False, True])
def test_pipeline_depth_and_lookahead_are_bitwise_neutral(dtype, causal):
    lib = _lib()
    B, H, N, d = 2, 3, 1000, 128       # ragged last tile; causal: the order across heads too
    scale = 1.0 / math.sqrt(d)
    q, k, v = (t.cuda().contiguous() for t in make_qkv(B, H, N, d, "bf16", seed=21))
    if dtype == "fp8":
        q, k, v, ds = fa.quantize_qkv_fp8(q, k, v)
        code, desc = fa.DTYPE_FP8_E4M3, ds.contiguous()
        o_ref, l_ref = fa.fwd(q, k, v, causal=causal, scale=scale, descales=desc, num_splits=1)
    else:
        code, desc = fa.DTYPE_BF16, None
        o_ref, l_ref = fa.fwd(q, k, v, causal=causal, scale=scale, num_splits=1)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream().cuda_stream
    for nstage in (2, 3):
        for look in (1, 2):
            for late in (0, 1):
                print(f"[case] {dtype} causal={causal} stages={nstage} look-ahead={look} late prefetch={late}",
                      flush=True)
                o = torch.empty_like(o_ref)
                lse = torch.empty_like(l_ref)
                rc = lib.fa_test_fwd_variant(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                             lse.data_ptr(), B, H, N, int(causal), scale, code,
                                             desc.data_ptr() if desc is not None else None, nstage, look, late,
                                             stream)
                assert rc == 0, rc
                torch.cuda.synchronize()
                assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), (dtype, causal, nstage, look, late)
                assert torch.equal(lse.view(torch.int32), l_ref.view(torch.int32)), (dtype, causal, nstage, look, late)
