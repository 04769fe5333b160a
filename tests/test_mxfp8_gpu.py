"""Per-block FP8 on the GPU, through the C ABI, against the fp64 oracle.

"Kernels and Memory in LLM Inference", section "Precision: FP8 with a real
failure mode": a scale per block so that an outlier coarsens only its own
block. Checked here:
  * fa_quantize_mxfp8_rows / _keys: codes and E8M0 scales byte-exact against
    oracle.quantize_mx (both sides take every decision in the same fp32
    arithmetic: the block max, a power-of-two scale, one RNE rounding), for
    bf16 and fp32 inputs, d = 64 and 128, ragged N, all-zero and tiny blocks,
    outlier inputs; the rotated variant against oracle.quantize_rotated_mx;
  * fa_fwd_mxfp8: O and L against the oracle's attention on the same
    dequantised values, with the FP8 tolerance (O 6e-2 plus the bf16 output
    floor, L 1e-3, cosine >= 0.999; on outlier inputs and on causal rows that
    see few keys the bound the multi-head FP8 tests derive from the
    arithmetic), causal and not, ragged N, GQA,
    split-KV, and on sampled rows of the DiT shape in the launch
    configuration bench.py times;
  * with unit scales everywhere the per-block kernel computes exactly what
    the per-head FP8 kernel computes with unit descales.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from fp8_bounds import assert_fp8
from tiled_attention_fa2_amd import fa
from tiled_attention_fa2_amd.inputs import make_gqa, make_qkv, make_signs, sample_rows

pytestmark = pytest.mark.gpu

TOL_O_FP8 = 6e-2
TOL_L = 1e-3


def _huddle(B, H, N, d, seed):
    """Values near 2^-10 with a few far out (the failure mode of one scale)."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((B, H, N, d), generator=g) * 2.0 ** -10
    out = torch.rand(x.shape, generator=g) < 1.0 / 512
    x[out] = 64.0
    return x.to(torch.bfloat16)


def _case_inputs(B, H, N, d, kind, seed, dtype="bf16"):
    if kind == "huddle":
        x = _huddle(B, H, N, d, seed)
        return x.float() if dtype == "f32" else x
    x, _, _ = make_qkv(B, H, N, d, dtype, seed=seed, variant=kind)
    if N > 3:
        x[0, 0, 2] = 0.0                         # an all-zero row
        x[0, -1, 1] *= 2.0 ** -110               # a tiny row (still normal after a 1/d fold)
    return x


QUANT_CASES = [(1, 3, 333, "iid"), (2, 2, 1, "iid"), (1, 2, 1000, "outlier"), (1, 1, 64, "peaked"),
               (1, 2, 100, "huddle"), (1, 1, 33, "iid")]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
def test_row_and_key_quantisers_byte_exact(dtype, d):
    for B, H, N, kind in QUANT_CASES:
        print(f"[case] {dtype} d={d} B={B} H={H} N={N} {kind}", flush=True)
        x = _case_inputs(B, H, N, d, kind, seed=N + d, dtype=dtype)
        xd = x.cuda()
        rc, rs = fa.quantize_mxfp8_rows(xd)
        kc, ks = fa.quantize_mxfp8_keys(xd)
        torch.cuda.synchronize()
        orc, ors = oracle.quantize_mx(x, "rows")
        okc, oks = oracle.quantize_mx(x, "keys")
        assert rs.shape == ors.shape and ks.shape == oks.shape
        assert np.array_equal(rs.cpu().numpy(), ors) and np.array_equal(rc.cpu().numpy(), orc)
        assert np.array_equal(ks.cpu().numpy(), oks) and np.array_equal(kc.cpu().numpy(), okc)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("fold", [False, True])
def test_rotated_row_quantiser_byte_exact(d, fold):
    s = make_signs(d, seed=3)
    for B, H, N, kind in QUANT_CASES:
        print(f"[case] rotated d={d} fold={fold} B={B} H={H} N={N} {kind}", flush=True)
        x = _case_inputs(B, H, N, d, kind, seed=2 * N + d)
        c, sc = fa.quantize_mxfp8_rows(x.cuda(), signs=s.cuda(), fold_inverse_d=fold)
        torch.cuda.synchronize()
        oc, osc = oracle.quantize_rotated_mx(x, s.numpy(), fold_inverse_d=fold)
        assert np.array_equal(sc.cpu().numpy(), osc) and np.array_equal(c.cpu().numpy(), oc)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_exponent_clamp_byte_exact(dtype):
    # magnitudes in [2^-122, 2^-121): the exponent that fits, -130, clamps to
    # -127 (every value stays a normal float, and x * 2^127 is exact)
    g = torch.Generator().manual_seed(13)
    mag = 1.0 + torch.rand((1, 2, 40, 128), generator=g)
    sign = 1 - 2 * torch.randint(0, 2, mag.shape, generator=g)
    x = (sign * mag * 2.0 ** -122).to(torch.bfloat16 if dtype == "bf16" else torch.float32)
    rc, rs = fa.quantize_mxfp8_rows(x.cuda())
    kc, ks = fa.quantize_mxfp8_keys(x.cuda())
    torch.cuda.synchronize()
    orc, ors = oracle.quantize_mx(x, "rows")
    okc, oks = oracle.quantize_mx(x, "keys")
    assert np.all(ors == 0) and np.all(oks == 0)
    assert np.array_equal(rs.cpu().numpy(), ors) and np.array_equal(rc.cpu().numpy(), orc)
    assert np.array_equal(ks.cpu().numpy(), oks) and np.array_equal(kc.cpu().numpy(), okc)


def test_fold_without_rotation_byte_exact():
    x = _case_inputs(1, 2, 77, 128, "iid", seed=4)
    c, sc = fa.quantize_mxfp8_rows(x.cuda(), fold_inverse_d=True)
    torch.cuda.synchronize()
    oc, osc = oracle.quantize_mx((x.float() * (1.0 / 128)).float(), "rows")
    assert np.array_equal(sc.cpu().numpy(), osc) and np.array_equal(c.cpu().numpy(), oc)


def _oracle_mx(q, k, v, scale, causal, rows=None, signs=None):
    if signs is None:
        qc, qs = oracle.quantize_mx(q, "rows")
        kc, ks = oracle.quantize_mx(k, "rows")
    else:
        qc, qs = oracle.quantize_rotated_mx(q, signs, True)
        kc, ks = oracle.quantize_rotated_mx(k, signs, False)
    vc, vs = oracle.quantize_mx(v, "keys")
    ref_in = (oracle.dequantize_mx(qc, qs, "rows"), oracle.dequantize_mx(kc, ks, "rows"),
              oracle.dequantize_mx(vc, vs, "keys"))
    if q.shape[1] != k.shape[1]:
        O, L = oracle.attention_gqa(*ref_in, scale=scale, causal=causal, rows=rows)
    else:
        O, L = oracle.attention(*ref_in, scale=scale, causal=causal, rows=rows)
    return O, L, ref_in


def _check(q, k, v, causal, scale, splits, label, outlier=False, signs=None):
    """Every case: O and L element by element within the bounds derived from
    the arithmetic (tests/fp8_bounds.py), cosine >= 0.999; iid inputs also
    within the FP8 tolerance on every row that averages at least 64 keys.
    outlier marks inputs that are not iid (outlier channels, huge |V|, the
    stress variants): they are held to the derived bounds alone."""
    print(f"[case] {label} shape={tuple(q.shape)} kv={tuple(k.shape)} causal={causal} splits={splits}", flush=True)
    sd = None if signs is None else signs.cuda()
    q8, k8, v8, sc = fa.quantize_qkv_mxfp8(q.cuda(), k.cuda(), v.cuda(), signs=sd)
    o, lse = fa.fwd_mxfp8(q8, k8, v8, sc, causal=causal, scale=scale, num_splits=splits)
    torch.cuda.synchronize()
    O_ref, L_ref, ref_in = _oracle_mx(q, k, v, scale, causal, signs=None if signs is None else signs.numpy())
    got_o = o.float().cpu().double().numpy()
    got_l = lse.cpu().double().numpy()
    floor = float(np.max(np.abs(torch.from_numpy(O_ref).to(torch.bfloat16).double().numpy() - O_ref)))
    err_o = float(np.max(np.abs(got_o - O_ref)))
    err_l = float(np.max(np.abs(got_l - L_ref)))
    print(f"    max|dO|={err_o:.3e} max|dL|={err_l:.3e} bf16-floor={floor:.3e}", flush=True)
    assert_fp8(got_o, got_l, O_ref, L_ref, ref_in, scale, causal=causal, label=label, iid=not outlier,
               floor=floor, tol_o=TOL_O_FP8, tol_l=TOL_L)


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_ragged_lengths(causal):
    for N in (1, 2, 37, 100, 129, 255, 700):
        q, k, v = make_qkv(2, 3, N, 128, "bf16", seed=N)
        _check(q, k, v, causal, 1 / math.sqrt(128), 1, f"ragged N={N}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("variant", ["outlier", "peaked", "growing"])
def test_fwd_stress_inputs(variant, causal):
    q, k, v = make_qkv(1, 4, 1000, 128, "bf16", seed=3, variant=variant)
    _check(q, k, v, causal, 1 / math.sqrt(128), 1, variant, outlier=True)


def test_fwd_huddle_inputs():
    # V holds outliers of 64: P's e4m3 rounding alone may move O by 2^-4 * 64,
    # so the bound derived from the arithmetic applies, not the O(1) tolerance
    q, k, v = (_huddle(1, 2, 600, 128, s) for s in (5, 6, 7))
    _check(q, k, v, False, 1 / math.sqrt(128), 1, "huddle", outlier=True)


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_split_and_gqa(causal):
    q, k, v = make_qkv(1, 2, 777, 128, "bf16", seed=8)
    _check(q, k, v, causal, 1 / math.sqrt(128), 3, "split 3")
    q, k, v = make_gqa(2, 8, 2, 300, 128, "bf16", seed=9)
    _check(q, k, v, causal, 1 / math.sqrt(128), 1, "gqa 8/2")
    _check(q, k, v, causal, 1 / math.sqrt(128), 2, "gqa 8/2 split 2")


def test_fwd_rotated_blocks():
    q, k, v = make_qkv(1, 3, 500, 128, "bf16", seed=10, variant="outlier")
    _check(q, k, v, False, 1 / math.sqrt(128), 1, "rotated + blocks", outlier=True, signs=make_signs(128, 2))


def test_unit_scales_match_the_per_head_kernel():
    # every block scale 2^0 and every descale 1: both kernels compute attention
    # of the same e4m3 values. With magnitudes 0.5 .. 1.875 (codes 0x30-0x3F)
    # every product is a multiple of 2^-8 and every score sum stays below 2^9,
    # so S is exact in fp32 in either kernel's summation order, and the rest
    # of the arithmetic is the same: the outputs agree bit for bit. The heads
    # are enough for the per-head forward to take its narrow tiles (more than
    # two workgroups per CU), which are the per-block kernel's tiles.
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    N, d = 300, 128
    B, H = 1, (2 * cus) // ((N + 127) // 128) + 1
    g = torch.Generator().manual_seed(11)
    codes = [(torch.randint(0x30, 0x40, (B, H, N, d), generator=g) |
              (torch.randint(0, 2, (B, H, N, d), generator=g) << 7)).to(torch.uint8) for _ in range(3)]
    q8, k8, v8 = (c.cuda() for c in codes)
    ones = torch.full((3, B * H), 1.0, device="cuda")
    unit = (torch.full((B, H, N, d // 32), 127, dtype=torch.uint8, device="cuda"),
            torch.full((B, H, N, d // 32), 127, dtype=torch.uint8, device="cuda"),
            torch.full((B, H, (N + 31) // 32, d), 127, dtype=torch.uint8, device="cuda"))
    o1, l1 = fa.fwd(q8, k8, v8, scale=0.01, descales=ones, num_splits=1)
    o2, l2 = fa.fwd_mxfp8(q8, k8, v8, unit, scale=0.01, num_splits=1)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention(*(oracle.e4m3_decode(c.numpy()) for c in codes), scale=0.01)
    assert float(np.max(np.abs(o2.float().cpu().double().numpy() - O_ref))) <= TOL_O_FP8
    assert float(np.max(np.abs(l2.cpu().double().numpy() - L_ref))) <= TOL_L
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_dit_shape_sampled_rows():
    # 56 heads x 30272 tokens x 128, the launch configuration bench.py times
    B, H, N, d = 1, 56, 30272, 128
    q, k, v = make_qkv(B, H, N, d, "bf16", seed=0)
    rows = sample_rows(N, tile=128, n_random=24)
    q8, k8, v8, sc = fa.quantize_qkv_mxfp8(q.cuda(), k.cuda(), v.cuda())
    o, lse = fa.fwd_mxfp8(q8, k8, v8, sc, scale=1 / math.sqrt(d), num_splits=1)
    torch.cuda.synchronize()
    heads = [0, 17, 55]
    O_ref, L_ref, ref_in = _oracle_mx(q[:, heads], k[:, heads], v[:, heads], 1 / math.sqrt(d), False, rows=rows)
    got_o = o[:, heads].float().cpu().double().numpy()[:, :, rows]
    got_l = lse[:, heads].cpu().double().numpy()[:, :, rows]
    err_o = float(np.max(np.abs(got_o - O_ref)))
    err_l = float(np.max(np.abs(got_l - L_ref)))
    print(f"[case] DiT sampled rows: max|dO|={err_o:.3e} max|dL|={err_l:.3e}", flush=True)
    assert err_o <= TOL_O_FP8 and err_l <= TOL_L
    assert_fp8(got_o, got_l, O_ref, L_ref, ref_in, 1 / math.sqrt(d), rows=rows, label="DiT sampled rows")


def test_bindings_reject_bad_arguments():
    x = torch.zeros((1, 1, 16, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        fa.quantize_mxfp8_rows(x, signs=torch.ones(32, dtype=torch.int8, device="cuda"))
    with pytest.raises(fa.FAError):
        fa.quantize_mxfp8_rows(x, signs=torch.ones(64, dtype=torch.int8, device="cuda"))   # fp32 + rotation
    q8 = torch.zeros((1, 1, 64, 64), dtype=torch.uint8, device="cuda")
    sc = (torch.zeros((1, 1, 64, 2), dtype=torch.uint8, device="cuda"),) * 2 + \
         (torch.zeros((1, 1, 2, 64), dtype=torch.uint8, device="cuda"),)
    with pytest.raises(fa.FAError):
        fa.fwd_mxfp8(q8, q8, q8, sc)                 # head dim 64 is not built
