"""Causal forward and backward with the work order that hands each XCD's
query tiles out longest first across its heads (2 x 8 heads, two per XCD; the
heads' K/V are far below the 32 MiB that selects that order), through the C
ABI:
  * against the fp64 oracle on every row (tolerances as in test_fwd_gpu:
    O 1e-5 fp32, 1e-2 bf16 plus the bf16 output floor, fp8 the bound derived
    from the arithmetic for causal rows with few keys; L 1e-3), unsplit and
    split into 3 key chunks;
  * bit-identical to launching each head alone (one head per launch takes the
    head-by-head order): the order moves work between workgroups, never the
    arithmetic of one (head, query tile).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from fp8_bounds import assert_fp8
from test_fwd_gpu import TOL_L, TOL_O, _metrics
from tiled_attention_fa2_amd import fa
from tiled_attention_fa2_amd.inputs import make_dout, make_qkv

pytestmark = pytest.mark.gpu

B, H, N, D = 2, 8, 777, 128


def _device_inputs(dtype, d=D):
    q, k, v = make_qkv(B, H, N, d, dtype, seed=41)
    if dtype != "fp8":
        return [t.cuda().contiguous() for t in (q, k, v)], None, (q, k, v)
    codes, ds = zip(*(oracle.quantize_per_head(t) for t in (q, k, v)))
    descales = torch.from_numpy(np.stack([d.ravel() for d in ds])).float().cuda().contiguous()
    dev = [torch.from_numpy(c).cuda().contiguous() for c in codes]
    ref_in = tuple(oracle.dequantize_per_head(c, d) for c, d in zip(codes, ds))
    return dev, descales, ref_in


@pytest.mark.parametrize("dtype", ["f32", "bf16", "fp8"])
@pytest.mark.parametrize("splits", [1, 3])
@pytest.mark.parametrize("d", [64, 128])
def test_causal_order_across_heads_forward(dtype, splits, d):
    print(f"[case] causal order across heads, fwd dtype={dtype} B={B} H={H} N={N} d={d} splits={splits}", flush=True)
    scale = 1.0 / math.sqrt(d)
    dev, descales, ref_in = _device_inputs(dtype, d)
    kw = dict(causal=True, scale=scale, num_splits=splits)
    if descales is not None:
        kw["descales"] = descales
    o, lse = fa.fwd(*dev, **kw)
    torch.cuda.synchronize()
    for b in range(B):
        for h in range(H):
            one = [t[b:b + 1, h:h + 1].contiguous() for t in dev]
            kw1 = dict(kw)
            if descales is not None:
                kw1["descales"] = descales[:, b * H + h].contiguous()
            o1, l1 = fa.fwd(*one, **kw1)
            torch.cuda.synchronize()
            assert torch.equal(o1, o[b:b + 1, h:h + 1]) and torch.equal(l1, lse[b:b + 1, h:h + 1]), (b, h)

    O_ref, L_ref = oracle.attention(*ref_in, scale=scale, causal=True)
    got_o = o.float().cpu().double().numpy()
    got_l = lse.cpu().double().numpy()
    err_o, cos, _, floor = _metrics(got_o, O_ref)
    err_l = float(np.max(np.abs(got_l - L_ref)))
    tol_o, tol_l = TOL_O[dtype] + (floor if dtype != "f32" else 0.0), TOL_L
    print(f"    max|dO|={err_o:.3e} max|dL|={err_l:.3e} cos={cos:.7f}", flush=True)
    assert np.all(np.isfinite(got_o)) and np.all(np.isfinite(got_l))
    if dtype == "fp8":
        # element by element within the derived bound; rows of >= 64 keys
        # within the FP8 tolerance
        assert_fp8(got_o, got_l, O_ref, L_ref, ref_in, scale, causal=True, label="causal order",
                   floor=floor)
    else:
        assert err_o <= tol_o and err_l <= tol_l


def test_causal_order_across_heads_backward():
    print(f"[case] causal order across heads, bwd B={B} H={H} N={N}", flush=True)
    q, k, v = (t.cuda().contiguous() for t in make_qkv(B, H, N, D, "bf16", seed=43))
    do = make_dout(B, H, N, D, seed=44).cuda().contiguous()
    o, lse = fa.fwd(q, k, v, causal=True, num_splits=1)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    for b in range(B):
        for h in range(H):
            one = [t[b:b + 1, h:h + 1].contiguous() for t in (q, k, v, o, lse, do)]
            g1 = fa.bwd(*one, causal=True)
            torch.cuda.synchronize()
            for got, full in zip(g1, (dq, dk, dv)):
                assert torch.equal(got, full[b:b + 1, h:h + 1]), (b, h)
