"""Parity of grouped-query attention (fa_fwd_gqa, through the C ABI) with the
fp64 oracle.

"Kernels and Memory in LLM Inference", section "Store less: MQA, GQA, MLA":
consecutive query heads share one key/value head; query head h reads K/V head
h / (Hq / Hkv). Checked here, for fp32, bf16 and fp8, head dims 64 and 128,
causal and not, unsplit and split-KV:
  * O and L against oracle.attention_gqa (the oracle fed the same fp8 codes);
  * bit-identity with the multi-head kernels run on K/V repeated head by head
    (the same arithmetic per query head, so the same bits);
  * the per-head quantiser on K/V heads, byte-exact against the oracle's.
Tolerances as for the multi-head forward: O 1e-5 / 1e-2 / 6e-2 (+ cosine
>= 0.999 for fp8), plus the bf16 rounding floor of the exact answer on these
non-workload shapes; L 1e-3.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from fp8_bounds import assert_fp8
from tiled_attention_fa2_amd import fa
from tiled_attention_fa2_amd.inputs import make_gqa, make_workload, sample_rows

pytestmark = pytest.mark.gpu

TOL_O = {"f32": 1e-5, "bf16": 1e-2, "fp8": 6e-2}
TOL_L = 1e-3


def _gqa_inputs(B, Hq, Hkv, N, d, dtype, seed):
    return make_gqa(B, Hq, Hkv, N, d, dtype, seed=seed)


def _device(q, k, v, dtype):
    if dtype == "fp8":
        codes, scales = zip(*(oracle.quantize_per_head(t) for t in (q, k, v)))
        descales = torch.from_numpy(np.concatenate([s.ravel() for s in scales])).cuda()
        dev = [torch.from_numpy(c).cuda().contiguous() for c in codes]
        ref = tuple(oracle.dequantize_per_head(c, s) for c, s in zip(codes, scales))
        return dev, descales, ref
    return [t.cuda().contiguous() for t in (q, k, v)], None, (q, k, v)


def _floor(O_ref):
    return float(np.max(np.abs(torch.from_numpy(O_ref).to(torch.bfloat16).double().numpy() - O_ref)))


@pytest.mark.parametrize("dtype", ["f32", "bf16", "fp8"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_gqa_matches_oracle(dtype, d, causal):
    for (Hq, Hkv), N, S in [((8, 2), 300, 1), ((6, 1), 777, 1), ((8, 2), 777, 3), ((4, 4), 129, 1)]:
        print(f"[case] dtype={dtype} d={d} causal={causal} Hq={Hq} Hkv={Hkv} N={N} splits={S}", flush=True)
        q, k, v = _gqa_inputs(1, Hq, Hkv, N, d, dtype, seed=N + Hq)
        dev, descales, ref = _device(q, k, v, dtype)
        o, lse = fa.fwd(*dev, causal=causal, scale=1.0 / math.sqrt(d), descales=descales, num_splits=S)
        torch.cuda.synchronize()
        O_ref, L_ref = oracle.attention_gqa(*ref, scale=1.0 / math.sqrt(d), causal=causal)
        got_o = o.float().cpu().double().numpy()
        got_l = lse.cpu().double().numpy()
        err_o = float(np.max(np.abs(got_o - O_ref)))
        err_l = float(np.max(np.abs(got_l - L_ref)))
        tol_o = TOL_O[dtype] + (_floor(O_ref) if dtype != "f32" else 0.0)
        print(f"    max|dO|={err_o:.3e} (tol {tol_o:.3e}) max|dL|={err_l:.3e}", flush=True)
        assert np.all(np.isfinite(got_o)) and np.all(np.isfinite(got_l))
        if dtype == "fp8":
            assert_fp8(got_o, got_l, O_ref, L_ref, ref, 1.0 / math.sqrt(d), causal=causal,
                       label=f"gqa {Hq}/{Hkv} N={N} splits={S}", floor=_floor(O_ref))
        else:
            assert err_o <= tol_o and err_l <= TOL_L


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("causal", [False, True])
def test_gqa_bit_identical_to_repeated_heads(dtype, causal):
    Hq, Hkv, N, d = 8, 2, 640, 128
    q, k, v = _gqa_inputs(2, Hq, Hkv, N, d, "bf16", seed=5)
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    kr = kd.repeat_interleave(Hq // Hkv, dim=1).contiguous()
    vr = vd.repeat_interleave(Hq // Hkv, dim=1).contiguous()
    for S in (1, 2):
        if dtype == "fp8":
            q8, k8, v8, ds = fa.quantize_qkv_fp8(qd, kd, vd)
            q8r, k8r, v8r, dsr = fa.quantize_qkv_fp8(qd, kr, vr)
            o1, l1 = fa.fwd(q8, k8, v8, causal=causal, descales=ds, num_splits=S)
            o2, l2 = fa.fwd(q8r, k8r, v8r, causal=causal, descales=dsr, num_splits=S)
        else:
            o1, l1 = fa.fwd(qd, kd, vd, causal=causal, num_splits=S)
            o2, l2 = fa.fwd(qd, kr, vr, causal=causal, num_splits=S)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2), (dtype, causal, S)


def test_gqa_quantiser_on_kv_heads_byte_exact():
    q, k, v = _gqa_inputs(2, 6, 2, 300, 64, "bf16", seed=9)
    q8, k8, v8, ds = fa.quantize_qkv_fp8(q.cuda(), k.cuda(), v.cuda())
    torch.cuda.synchronize()
    assert ds.shape == (2 * 6 + 2 * 2 * 2,)
    off = 0
    for t, t8 in ((q, q8), (k, k8), (v, v8)):
        codes, scales = oracle.quantize_per_head(t)
        n = scales.size
        assert np.array_equal(t8.cpu().numpy(), codes)
        assert np.array_equal(ds[off:off + n].cpu().numpy(), scales.ravel().astype(np.float32))
        off += n


def test_gqa_workload_sampled_rows():
    # the benchmark's GQA workload (56 query heads over 8 K/V heads, 30272
    # tokens) in the launch configuration bench.py times, on sampled rows
    w, (q, k, v) = make_workload("bf16_gqa_b1_hq56_hkv8_n30272_d128", seed=0)
    rows = sample_rows(w.N, tile=128, n_random=32)
    o, lse = fa.fwd(q.cuda(), k.cuda(), v.cuda(), causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention_gqa(q, k, v, scale=w.scale, causal=w.causal, rows=rows)
    got_o = o.float().cpu().double().numpy()[:, :, rows]
    got_l = lse.cpu().double().numpy()[:, :, rows]
    err_o = float(np.max(np.abs(got_o - O_ref)))
    err_l = float(np.max(np.abs(got_l - L_ref)))
    print(f"[case] {w.name}: max|dO|={err_o:.3e} max|dL|={err_l:.3e}", flush=True)
    assert err_o <= TOL_O["bf16"] and err_l <= TOL_L


def test_gqa_rejects_indivisible_heads():
    q, k, v = _gqa_inputs(1, 6, 4, 64, 64, "bf16", seed=1)
    with pytest.raises(ValueError):
        fa.fwd(q.cuda(), k.cuda(), v.cuda())
