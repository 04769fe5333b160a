"""Rotation before FP8 quantisation on the GPU (fa_quantize_fp8_rotated and
the FP8 forward on its codes), through the C ABI, against the fp64 oracle.

"Kernels and Memory in LLM Inference", section "Precision: FP8 with a real
failure mode": Q and K are multiplied by one fixed random rotation before FP8
quantisation, which spreads outlier coordinates over all dimensions; the
rotations cancel in Q K^T. Checked here:
  * codes and descales byte-exact against oracle.quantize_rotated (the
    rotated values are exact sums rounded once to fp32 on both sides, and the
    quantiser takes its decisions in fp32 on both sides), for d = 64 and 128,
    ragged and single-row heads, all-zero heads, outlier inputs, and both
    settings of the folded 1/d;
  * the FP8 forward on rotated codes against the oracle's attention on the
    same dequantised codes (the FP8 tolerance, O 6e-2 and cosine >= 0.999; on
    outlier inputs the bound derived for them in the multi-head FP8 tests);
  * what the rotation is for: on inputs with outlier channels the attention
    error against the exact bf16 answer falls well below that of plain FP8,
    and on plain Gaussian inputs it is no worse.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from fp8_bounds import assert_fp8
from tiled_attention_fa2_amd import fa
from tiled_attention_fa2_amd.inputs import make_qkv, make_signs

pytestmark = pytest.mark.gpu

TOL_O_FP8 = 6e-2


def _signs(d, seed=1):
    return make_signs(d, seed=seed)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("fold", [False, True])
def test_rotated_codes_byte_exact(d, fold):
    s = _signs(d)
    sd = s.cuda()
    for B, H, N, variant in [(1, 3, 333, "iid"), (2, 2, 1, "iid"), (1, 2, 1000, "outlier"),
                             (1, 1, 64, "peaked")]:
        print(f"[case] d={d} fold={fold} B={B} H={H} N={N} {variant}", flush=True)
        x, _, _ = make_qkv(B, H, N, d, "bf16", seed=N + d, variant=variant)
        codes, desc = fa.quantize_fp8_rotated(x.cuda(), sd, fold)
        torch.cuda.synchronize()
        ref_codes, ref_desc = oracle.quantize_rotated(x, s.numpy(), fold_inverse_d=fold)
        got = codes.cpu().numpy()
        n_diff = int(np.count_nonzero(got != ref_codes))
        print(f"    differing codes: {n_diff}", flush=True)
        assert n_diff == 0
        assert np.array_equal(desc.cpu().numpy(), ref_desc.ravel().astype(np.float32))


def test_rotated_zero_head_and_empty():
    d = 128
    s = _signs(d, seed=4)
    x, _, _ = make_qkv(1, 3, 200, d, "bf16", seed=2)
    x[0, 1] = 0.0
    codes, desc = fa.quantize_fp8_rotated(x.cuda(), s.cuda(), True)
    torch.cuda.synchronize()
    ref_codes, ref_desc = oracle.quantize_rotated(x, s.numpy(), fold_inverse_d=True)
    assert np.array_equal(codes.cpu().numpy(), ref_codes)
    assert np.array_equal(desc.cpu().numpy(), ref_desc.ravel().astype(np.float32))
    assert desc[1].item() == 1.0 / d
    # no rows: descales are still written (1, times the folded 1/d)
    e = torch.empty((2, 2, 0, d), dtype=torch.bfloat16, device="cuda")
    c0, d0 = fa.quantize_fp8_rotated(e, s.cuda(), True)
    torch.cuda.synchronize()
    assert c0.numel() == 0 and torch.equal(d0.cpu(), torch.full((4,), 1.0 / d))


def test_all_plus_signs_is_the_plain_hadamard():
    # s = +1 everywhere: the code of row e_j (a basis vector) is the j-th row
    # of H, every entry +-1, so every code is +-448's code and the descale 1/448
    d = 64
    x = torch.zeros((1, 1, d, d), dtype=torch.bfloat16)
    x[0, 0] = torch.eye(d, dtype=torch.bfloat16)
    codes, desc = fa.quantize_fp8_rotated(x.cuda(), torch.ones(d, dtype=torch.int8, device="cuda"), False)
    torch.cuda.synchronize()
    H = oracle.hadamard(d)
    c = codes.cpu().numpy()[0, 0]
    assert np.array_equal(c == 0x7E, H > 0) and np.array_equal(c == 0xFE, H < 0)
    assert desc.item() == np.float32(1.0) / np.float32(448.0)


@pytest.mark.parametrize("variant", ["iid", "outlier"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_fwd_on_rotated_codes_matches_oracle(variant, causal, d):
    # iid inputs: the FP8 tolerance on rows that average many keys, and the
    # per-element bound derived from the arithmetic everywhere; outlier inputs
    # (|V| up to ~80): the derived bound alone

    B, H, N = 1, 3, 700
    q, k, v = make_qkv(B, H, N, d, "bf16", seed=17 + d, variant=variant)
    s = _signs(d, seed=5)
    q8, k8, v8, desc = fa.quantize_qkv_fp8(q.cuda(), k.cuda(), v.cuda(), signs=s.cuda())
    for S in (1, 3):
        print(f"[case] causal={causal} d={d} splits={S}", flush=True)
        o, lse = fa.fwd(q8, k8, v8, causal=causal, scale=1.0 / math.sqrt(d), descales=desc, num_splits=S)
        torch.cuda.synchronize()
        cq, dq = oracle.quantize_rotated(q, s.numpy(), fold_inverse_d=True)
        ck, dk = oracle.quantize_rotated(k, s.numpy(), fold_inverse_d=False)
        cv, dv = oracle.quantize_per_head(v)
        assert np.array_equal(q8.cpu().numpy(), cq) and np.array_equal(k8.cpu().numpy(), ck)
        ref_in = (oracle.dequantize_per_head(cq, dq), oracle.dequantize_per_head(ck, dk),
                  oracle.dequantize_per_head(cv, dv))
        O_ref, L_ref = oracle.attention(*ref_in, 1.0 / math.sqrt(d), causal=causal)
        got_o = o.float().cpu().double().numpy()
        got_l = lse.cpu().double().numpy()
        floor = float(np.max(np.abs(torch.from_numpy(O_ref).to(torch.bfloat16).double().numpy() - O_ref)))
        err_o = float(np.max(np.abs(got_o - O_ref)))
        err_l = float(np.max(np.abs(got_l - L_ref)))
        print(f"    max|dO|={err_o:.3e} max|dL|={err_l:.3e}", flush=True)
        assert_fp8(got_o, got_l, O_ref, L_ref, ref_in, 1.0 / math.sqrt(d), causal=causal,
                   label=f"rotated {variant} splits={S}", iid=variant == "iid", floor=floor, tol_o=TOL_O_FP8)


def _rms(a, b):
    return float(np.sqrt(np.mean((a - b) ** 2)))


@pytest.mark.parametrize("variant,ratio", [("outlier", 0.5), ("iid", 1.1)])
def test_rotation_reduces_fp8_error(variant, ratio):
    # error of the FP8 forward against the exact attention of the bf16 inputs,
    # plain per-head FP8 versus rotated FP8 (measured on the oracle: outlier
    # inputs about 0.28x, Gaussian inputs about 1x)
    B, H, N, d = 1, 4, 1024, 128
    q, k, v = make_qkv(B, H, N, d, "bf16", seed=23, variant=variant)
    scale = 1.0 / math.sqrt(d)
    O_exact, _ = oracle.attention(q, k, v, scale)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    p8 = fa.quantize_qkv_fp8(qd, kd, vd)
    r8 = fa.quantize_qkv_fp8(qd, kd, vd, signs=_signs(d, seed=9).cuda())
    o_plain, _ = fa.fwd(*p8[:3], scale=scale, descales=p8[3])
    o_rot, _ = fa.fwd(*r8[:3], scale=scale, descales=r8[3])
    torch.cuda.synchronize()
    e_plain = _rms(o_plain.float().cpu().double().numpy(), O_exact)
    e_rot = _rms(o_rot.float().cpu().double().numpy(), O_exact)
    print(f"[case] {variant}: rms error plain {e_plain:.4e} rotated {e_rot:.4e}", flush=True)
    assert e_rot <= ratio * e_plain


def test_rotated_quantiser_rejects_bad_arguments():
    x = torch.zeros((1, 1, 16, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(TypeError):
        fa.quantize_fp8_rotated(x, torch.ones(64, dtype=torch.int8, device="cuda"), False)
    with pytest.raises(ValueError):
        fa.quantize_fp8_rotated(x.bfloat16(), torch.ones(32, dtype=torch.int8, device="cuda"), False)
