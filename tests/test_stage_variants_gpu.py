"""Determinism across pipeline depths: the race detector.

The forward kernel fa_fwd launches for bf16 and FP8, at head dim 128 in both
of its tile configurations (narrow: key tile 32 / 64, three waves per SIMD,
for full grids; wide: 64 / 128, two waves per SIMD, for grids of at most two
workgroups per CU) and at head dim 64 (key tile 64 / 128, four / three waves
per SIMD), is built again by tests/hip/stage_variants.hip with 2 and 3 LDS stages, with MFMA operand reads 1 and 2 steps ahead, and with each
tile's prefetch issued before or after its QK MFMAs. None of these changes
which values are added in which order; they change only when K/V tiles land in
LDS and when operands are read. So every variant must reproduce the library's
own configuration bit for bit: a missing wait or barrier (a tile read before
it landed, or overwritten while a slower wave still reads it) would show up as
a difference.

Each baseline is also held to the oracle (bf16: 1e-2 plus the bf16 floor;
FP8: the per-element bounds), on ragged and one-key shapes, and must equal
fa_fwd bit for bit on a grid for which fa_fwd picks that configuration.
"""
import ctypes
import math
import os

import numpy as np
import pytest
import torch

import oracle
from fp8_bounds import assert_fp8
from tiled_attention_fa2_amd import fa
from tiled_attention_fa2_amd.inputs import make_qkv

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "tests", "hip", "libstage_variants.so")
# configurations: 0 = head dim 128 narrow, 1 = head dim 128 wide, 2 = head dim 64
CFG_D = {0: 128, 1: 128, 2: 64}
# the library's choices: (dtype, cfg) -> (stages, look-ahead, late prefetch), causal or not
LIBRARY = {("bf16", 0): (3, 2, 0), ("fp8", 0): (2, 2, 0),
           ("bf16", 1): (2, 2, 0), ("fp8", 1): (2, 2, 0),
           ("bf16", 2): (2, 2, 0), ("fp8", 2): (2, 2, 0)}


def _lib():
    if not os.path.exists(LIB):
        pytest.fail("tests/hip/libstage_variants.so is not built (python -m tiled_attention_fa2_amd.build)")
    lib = ctypes.CDLL(LIB)
    lib.fa_test_fwd_variant.restype = ctypes.c_int
    lib.fa_test_fwd_variant.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 5 + [ctypes.c_float, ctypes.c_int,
                                        ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_void_p]
    return lib


def _inputs(dtype, B, H, N, seed, d=128):
    q, k, v = (t.cuda().contiguous() for t in make_qkv(B, H, N, d, "bf16", seed=seed))
    if dtype == "fp8":
        q, k, v, ds = fa.quantize_qkv_fp8(q, k, v)
        return (q, k, v), ds.contiguous()
    return (q, k, v), None


def _variant(lib, qkv, desc, dtype, causal, scale, cfg, nstage, look, late):
    q, k, v = qkv
    B, H, N, d = q.shape
    assert d == CFG_D[cfg]
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    code = fa.DTYPE_FP8_E4M3 if dtype == "fp8" else fa.DTYPE_BF16
    rc = lib.fa_test_fwd_variant(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, N,
                                 d, int(causal), scale, code, desc.data_ptr() if desc is not None else None, nstage,
                                 look, late, int(cfg == 1), torch.cuda.current_stream().cuda_stream)
    assert rc == 0, rc
    torch.cuda.synchronize()
    return o, lse


def _check_oracle(o, lse, qkv, desc, dtype, causal, scale, label):
    B, H = qkv[0].shape[:2]
    if dtype == "fp8":
        ds = desc.cpu().numpy().reshape(3, B, H)
        ref_in = tuple(oracle.dequantize_per_head(t.cpu().numpy(), ds[i]) for i, t in enumerate(qkv))
        O, L = oracle.attention(*ref_in, scale=scale, causal=causal)
        assert_fp8(o.float().cpu().numpy(), lse.cpu().numpy(), O, L, ref_in, scale, causal=causal, label=label)
    else:
        ref_in = tuple(t.double().cpu().numpy() for t in qkv)
        O, L = oracle.attention(*ref_in, scale=scale, causal=causal)
        floor = float(np.max(np.abs(torch.from_numpy(O).to(torch.bfloat16).double().numpy() - O)))
        assert np.max(np.abs(o.double().cpu().numpy() - O)) <= 1e-2 + floor, label
        assert np.max(np.abs(lse.double().cpu().numpy() - L)) <= 1e-3, label


@pytest.mark.parametrize("cfg", [0, 1, 2])
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("causal", [False, True])
def test_pipeline_depth_and_lookahead_are_bitwise_neutral(dtype, causal, cfg):
    lib = _lib()
    B, H, N, d = 2, 3, 1000, CFG_D[cfg]     # ragged last tile; causal: the order across heads too
    scale = 1.0 / math.sqrt(d)
    qkv, desc = _inputs(dtype, B, H, N, seed=21, d=d)
    base = LIBRARY[(dtype, cfg)]
    o_ref, l_ref = _variant(lib, qkv, desc, dtype, causal, scale, cfg, *base)
    _check_oracle(o_ref, l_ref, qkv, desc, dtype, causal, scale, f"{dtype} causal={causal} cfg={cfg}")
    for nstage in (2, 3):
        for look in (1, 2):
            for late in (0, 1):
                print(f"[case] {dtype} causal={causal} cfg={cfg} stages={nstage} look-ahead={look} "
                      f"late prefetch={late}", flush=True)
                o, lse = _variant(lib, qkv, desc, dtype, causal, scale, cfg, nstage, look, late)
                key = (dtype, causal, cfg, nstage, look, late)
                assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), key
                assert torch.equal(lse.view(torch.int32), l_ref.view(torch.int32)), key


@pytest.mark.parametrize("cfg", [0, 1, 2])
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_every_configuration_on_edge_shapes(dtype, cfg):
    # one key, a single partial tile, one tile plus one key, causal and not
    lib = _lib()
    scale = 0.3
    for N in (1, 33, 129):
        qkv, desc = _inputs(dtype, 1, 2, N, seed=N, d=CFG_D[cfg])
        for causal in (False, True):
            o, lse = _variant(lib, qkv, desc, dtype, causal, scale, cfg, *LIBRARY[(dtype, cfg)])
            _check_oracle(o, lse, qkv, desc, dtype, causal, scale, f"{dtype} N={N} causal={causal} cfg={cfg}")


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_baselines_are_the_library(dtype):
    # at head dim 128 fa_fwd picks the wide tiles for a grid of at most two
    # workgroups per CU and the narrow ones above; head dim 64 has one
    # configuration; compared on the unsplit path
    lib = _lib()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    N = 1000
    scale = 1.0 / math.sqrt(128)
    for H, cfg in ((3, 1), ((2 * cus) // ((N + 127) // 128) + 1, 0), (3, 2)):
        qkv, desc = _inputs(dtype, 1, H, N, seed=22, d=CFG_D[cfg])
        if cfg < 2:
            assert (H * ((N + 127) // 128) <= 2 * cus) == (cfg == 1)
        o_ref, l_ref = _variant(lib, qkv, desc, dtype, False, scale, cfg, *LIBRARY[(dtype, cfg)])
        kw = dict(descales=desc) if dtype == "fp8" else {}
        o, lse = fa.fwd(*qkv, scale=scale, num_splits=1, **kw)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), (dtype, H, cfg)
        assert torch.equal(lse.view(torch.int32), l_ref.view(torch.int32)), (dtype, H, cfg)
