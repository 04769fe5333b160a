"""The forward at a long sequence, through the C ABI, against the fp64 oracle
on sampled rows: one head of 262181 tokens (2048 query tiles and a ragged
tail), so every byte offset inside a head reaches 67 MB (the kernels address
one head with 32-bit buffer offsets) and the key loop runs 8194 / 4097 tiles.
bf16 and fp8 (the per-head quantiser on the device, the oracle fed the same
codes), causal and not, unsplit and split into key chunks.

Rows checked: 0, 1, N-1, the whole last (ragged) query tile and 24 uniform
draws. Tolerances: O 1e-2 (bf16) / 6e-2 plus cosine >= 0.999 (fp8), plus the
bf16 output floor, L 1e-3; fp8 causal takes the bound derived from the
arithmetic (its first rows average one or two keys).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from fp8_bounds import assert_fp8
from tiled_attention_fa2_amd import fa
from tiled_attention_fa2_amd.inputs import make_qkv, sample_rows

pytestmark = pytest.mark.gpu

N_LONG = 262144 + 37
TOL_O = {"bf16": 1e-2, "fp8": 6e-2}
TOL_L = 1e-3


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("causal", [False, True])
def test_long_sequence_sampled_rows(dtype, causal):
    d = 128
    scale = 1.0 / math.sqrt(d)
    q, k, v = make_qkv(1, 1, N_LONG, d, "bf16", seed=31)
    rows = sample_rows(N_LONG, tile=128, n_random=24)
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    if dtype == "fp8":
        q8, k8, v8, ds = fa.quantize_qkv_fp8(qd, kd, vd)
        torch.cuda.synchronize()
        codes = [t.cpu().numpy() for t in (q8, k8, v8)]
        dsc = ds.cpu().numpy().reshape(3, 1, 1)
        # the oracle's own quantiser must give the same codes (both decide in fp32)
        for c, t in zip(codes, (q, k, v)):
            assert np.array_equal(c, oracle.quantize_per_head(t)[0])
        ref_in = [oracle.dequantize_per_head(c, dsc[i]) for i, c in enumerate(codes)]
        args, kw = (q8, k8, v8), dict(descales=ds)
    else:
        ref_in = [q, k, v]
        args, kw = (qd, kd, vd), {}
    O_ref, L_ref = oracle.attention(*ref_in, scale=scale, causal=causal, rows=rows)
    for splits in (1, 3):
        print(f"[case] N={N_LONG} {dtype} causal={causal} splits={splits}", flush=True)
        o, lse = fa.fwd(*args, causal=causal, scale=scale, num_splits=splits, **kw)
        torch.cuda.synchronize()
        got_o = o.float().cpu().double().numpy()[:, :, rows]
        got_l = lse.cpu().double().numpy()[:, :, rows]
        err_o = float(np.max(np.abs(got_o - O_ref)))
        err_l = float(np.max(np.abs(got_l - L_ref)))
        a, b = got_o.ravel(), O_ref.ravel()
        cos = float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))
        floor = float(np.max(np.abs(torch.from_numpy(O_ref).to(torch.bfloat16).double().numpy() - O_ref)))
        tol_o, tol_l = TOL_O[dtype] + floor, TOL_L
        print(f"    max|dO|={err_o:.3e} max|dL|={err_l:.3e} cos={cos:.7f}", flush=True)
        assert np.all(np.isfinite(got_o)) and np.all(np.isfinite(got_l))
        if dtype == "fp8":
            # causal rows 0 and 1 average one or two keys, where P's e4m3
            # rounding is not averaged out: every element within the bound
            # derived from the arithmetic, rows of >= 64 keys within 6e-2
            assert_fp8(got_o, got_l, O_ref, L_ref, ref_in, scale, causal=causal, rows=rows,
                       label=f"N={N_LONG} splits={splits}", floor=floor)
        else:
            assert err_o <= tol_o and err_l <= tol_l
