"""Parity of the split-KV path with the fp64 oracle, through the C ABI.

fa_fwd_splitkv cuts the keys into chunks of fa_splitkv_chunk_keys(N, S) keys
("Kernels and Memory in LLM Inference", section "Flash-Decoding: one token,
whole chip"), writes one partial result per chunk into the caller's workspace
and merges them. Checked here:
  * every partial in the workspace against oracle.attention_keyrange over the
    same key chunk (rows with no valid key in the chunk must be exactly
    L = -inf, O = 0);
  * the merged O and L against oracle.attention;
  * fa_merge_partials alone against oracle.merge_partials on seeded partials
    with empty parts, empty rows and weights 500 nats apart;
  * the default path (the library's own choice of splits) on the 8-head
    4096-token workload, and a 2-way split of the 56-head 30272-token one on
    sampled rows.
Tolerances as for the unsplit forward: O 1e-5 (fp32) / 1e-2 (bf16) / 6e-2 and
cosine >= 0.999 (fp8); L 1e-3. The partials are fp32 (no output rounding);
the merged bf16 O adds the bf16 rounding floor of the exact answer on the
non-workload cases.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from fp8_bounds import assert_fp8
from tiled_attention_fa2_amd import fa
from tiled_attention_fa2_amd.inputs import WORKLOADS, make_partials, make_qkv, sample_rows

pytestmark = pytest.mark.gpu

TOL_O = {"f32": 1e-5, "bf16": 1e-2, "fp8": 6e-2}
TOL_L = 1e-3


def _device_inputs(q, k, v, dtype):
    """Device tensors (+ descales) for the GPU and the exact fp64 inputs the
    oracle must see."""
    if dtype == "fp8":
        c_q, ds_q = oracle.quantize_per_head(q)
        c_k, ds_k = oracle.quantize_per_head(k)
        c_v, ds_v = oracle.quantize_per_head(v)
        descales = torch.from_numpy(np.stack([ds_q.ravel(), ds_k.ravel(), ds_v.ravel()])).cuda()
        dev = [torch.from_numpy(c).cuda().contiguous() for c in (c_q, c_k, c_v)]
        ref = (oracle.dequantize_per_head(c_q, ds_q), oracle.dequantize_per_head(c_k, ds_k),
               oracle.dequantize_per_head(c_v, ds_v))
        return dev, descales, ref
    return [t.cuda().contiguous() for t in (q, k, v)], None, (q, k, v)


def _bf16_floor(O_ref):
    return float(np.max(np.abs(torch.from_numpy(O_ref).to(torch.bfloat16).double().numpy() - O_ref)))


def _cos(a, b):
    a = a.ravel()
    b = b.ravel()
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b) + 1e-300))


def _check_split(q, k, v, dtype, causal, scale, S, label, rows=None, check_parts=True, extra=True, iid=True):
    B, H, N, d = q.shape
    print(f"[case] {label} dtype={dtype} shape={tuple(q.shape)} causal={causal} splits={S}", flush=True)
    dev, descales, ref = _device_inputs(q, k, v, dtype)
    need = fa.splitkv_workspace_bytes(B, H, N, d, S)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    o, lse = fa.fwd(*dev, causal=causal, scale=scale, descales=descales, num_splits=S, workspace=ws)
    torch.cuda.synchronize()
    chunk = fa.splitkv_chunk_keys(N, S)
    used = -(-N // chunk)
    assert chunk % 128 == 0 and 1 <= used <= S

    if check_parts:
        o_parts, lse_parts = fa.splitkv_partials(ws, S, B, H, N, d)
        for s in range(used):
            O_s, L_s = oracle.attention_keyrange(*ref, scale, causal, s * chunk, (s + 1) * chunk, rows=rows)
            got_o = o_parts[s].cpu().double().numpy().reshape(B, H, N, d)
            got_l = lse_parts[s].cpu().double().numpy().reshape(B, H, N)
            if rows is not None:
                got_o, got_l = got_o[:, :, rows], got_l[:, :, rows]
            empty = ~np.isfinite(L_s)
            assert np.array_equal(got_l == -np.inf, empty), (label, s, "empty rows differ")
            assert np.all(got_o[empty] == 0.0), (label, s)
            full = ~empty
            err_o = float(np.max(np.abs(got_o - O_s)[full], initial=0.0))
            err_l = float(np.max(np.abs(got_l[full] - L_s[full]), initial=0.0))
            print(f"    chunk {s} keys [{s * chunk}, {min(N, (s + 1) * chunk)}) rows with keys "
                  f"{int(full.sum())}: max|dO|={err_o:.3e} max|dL|={err_l:.3e}", flush=True)
            assert np.all(np.isfinite(got_o)) and np.all(np.isfinite(got_l[full]))
            if dtype == "fp8":
                # the chunk's partial against the oracle on the chunk's keys,
                # element by element within the derived bound
                assert_fp8(got_o, got_l, O_s, L_s, ref, scale, causal=causal, rows=rows,
                           key_range=(s * chunk, (s + 1) * chunk), label=f"{label} chunk {s}", iid=iid)
            else:
                assert err_o <= TOL_O[dtype], (label, s, err_o)
                assert err_l <= TOL_L, (label, s, err_l)

    O_ref, L_ref = oracle.attention(*ref, scale=scale, causal=causal, rows=rows)
    got_o = o.float().cpu().double().numpy()
    got_l = lse.cpu().double().numpy()
    if rows is not None:
        got_o, got_l = got_o[:, :, rows], got_l[:, :, rows]
    err_o = float(np.max(np.abs(got_o - O_ref)))
    err_l = float(np.max(np.abs(got_l - L_ref)))
    floor = _bf16_floor(O_ref) if (extra and dtype != "f32") else 0.0
    print(f"    merged: max|dO|={err_o:.3e} max|dL|={err_l:.3e} cos={_cos(got_o, O_ref):.6f}", flush=True)
    assert np.all(np.isfinite(got_o)) and np.all(np.isfinite(got_l))
    if dtype == "fp8":
        assert_fp8(got_o, got_l, O_ref, L_ref, ref, scale, causal=causal, rows=rows, label=f"{label} merged",
                   iid=iid, floor=floor)
        if not extra:
            assert err_o <= TOL_O[dtype] and err_l <= TOL_L, (label, err_o, err_l)
    else:
        assert err_o <= TOL_O[dtype] + floor, (label, err_o)
        assert err_l <= TOL_L, (label, err_l)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "fp8"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_split_partials_and_merge(dtype, d, causal):
    # N = 777: a ragged last tile and chunks of several key tiles each;
    # S = 5 leaves chunks of 256 keys (4 written); N = 129, S = 2: a one-key chunk
    for N, S in [(777, 2), (777, 3), (777, 5), (129, 2)]:
        q, k, v = make_qkv(1, 2, N, d, dtype, seed=N + S)
        _check_split(q, k, v, dtype, causal, 1.0 / math.sqrt(d), S, label=f"N={N} d={d}")


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_split_stress_inputs(dtype):
    # running max rising every tile, and near one-hot rows, across chunk borders
    for variant in ("growing", "peaked"):
        q, k, v = make_qkv(1, 2, 600, 128, dtype, seed=3, variant=variant)
        for causal in (False, True):
            _check_split(q, k, v, dtype, causal, 1.0 / math.sqrt(128), 3, label=variant, iid=False)


def test_split_one_chunk_equals_whole():
    # num_splits = 1 through the split path: one chunk of every key
    q, k, v = make_qkv(2, 2, 300, 128, "bf16", seed=11)
    _check_split(q, k, v, "bf16", True, 1.0 / math.sqrt(128), 1, label="S=1")


def test_default_path_on_8_head_workload():
    w = WORKLOADS["bf16_b1_h8_n4096_d128"]
    S = fa.default_splits(w.B, w.H, w.N, w.d, w.causal, fa.DTYPE_BF16)
    print(f"default splits for {w.name}: {S}", flush=True)
    assert S > 1  # 256 workgroups cannot fill a 256-CU device three deep
    q, k, v = make_qkv(w.B, w.H, w.N, w.d, w.dtype, seed=0)
    _check_split(q, k, v, w.dtype, w.causal, w.scale, S, label=w.name, check_parts=False, extra=False)
    # and fwd() with no num_splits takes that path with the same result
    dev = [t.cuda() for t in (q, k, v)]
    ws = torch.empty(fa.splitkv_workspace_bytes(w.B, w.H, w.N, w.d, S), dtype=torch.uint8, device="cuda")
    o1, l1 = fa.fwd(*dev, scale=w.scale, num_splits=S, workspace=ws)
    o2, l2 = fa.fwd(*dev, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("name", ["bf16_dit_b1_h56_n30272_d128", "fp8_dit_b1_h56_n30272_d128"])
def test_two_way_split_at_full_size(name):
    w = WORKLOADS[name]
    q, k, v = make_qkv(w.B, w.H, w.N, w.d, w.dtype, seed=0)
    rows = sample_rows(w.N, tile=128, n_random=16)
    _check_split(q, k, v, w.dtype, w.causal, w.scale, 2, label=name, rows=rows, extra=False)


@pytest.mark.parametrize("S", [1, 2, 5])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_merge_kernel(S, d, out_dtype):
    o_parts, lse_parts = make_partials(S, 3, 257, d, seed=S * 1000 + d)
    print(f"[case] merge S={S} d={d} out={out_dtype}", flush=True)
    o, lse = fa.merge_partials(o_parts.cuda(), lse_parts.cuda(), out_dtype)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.merge_partials(o_parts.double().numpy(), lse_parts.double().numpy())
    got_o = o.float().cpu().double().numpy()
    got_l = lse.cpu().double().numpy()
    empty = ~np.isfinite(L_ref)
    assert np.array_equal(got_l == -np.inf, empty)
    assert np.all(got_o[empty] == 0.0)
    full = ~empty
    # fp32 arithmetic: a few ulps of |O| and of |L| (L reaches ~550 here)
    tol_o = 1e-5 * max(1.0, float(np.max(np.abs(O_ref)))) + \
        (_bf16_floor(O_ref) if out_dtype == torch.bfloat16 else 0.0)
    err_o = float(np.max(np.abs(got_o - O_ref)))
    err_l = float(np.max(np.abs(got_l[full] - L_ref[full])))
    tol_l = 4e-7 * max(1.0, float(np.max(np.abs(L_ref[full])))) + 1e-6
    print(f"    max|dO|={err_o:.3e} (tol {tol_o:.3e})  max|dL|={err_l:.3e} (tol {tol_l:.3e})", flush=True)
    assert err_o <= tol_o and err_l <= tol_l


def test_split_errors_raise():
    q, k, v = make_qkv(1, 1, 256, 128, "bf16", seed=1)
    dev = [t.cuda() for t in (q, k, v)]
    small = torch.empty(fa.splitkv_workspace_bytes(1, 1, 256, 128, 2) - 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(fa.FAError) as e:
        fa.fwd(*dev, num_splits=2, workspace=small)
    assert e.value.status == -9
    with pytest.raises(fa.FAError) as e:
        fa.fwd(*dev, num_splits=fa.FA_MAX_SPLITS + 1)
    assert e.value.status == -10


def test_caller_workspace_is_checked_on_every_path():
    """A caller's workspace reaches the library with its own size, so one that
    is too small is refused (FA_ERR_WORKSPACE, before any launch) on the
    split-KV, grouped-query, per-block FP8 and backward paths; one that is not
    a contiguous uint8 device tensor is refused by the binding."""
    print("[case] caller workspaces: too small / wrong dtype on fwd, gqa, mxfp8, bwd", flush=True)
    N, d = 256, 128
    q, k, v = (t.cuda() for t in make_qkv(1, 2, N, d, "bf16", seed=2))
    need = fa.splitkv_workspace_bytes(1, 2, N, d, 2)
    small = torch.empty(need - 16, dtype=torch.uint8, device="cuda")
    wrong = torch.empty(need // 4 + 16, dtype=torch.float32, device="cuda")
    k1, v1 = k[:, :1].contiguous(), v[:, :1].contiguous()
    m8 = fa.quantize_qkv_mxfp8(q, k, v)
    calls = [
        ("fwd split", lambda ws: fa.fwd(q, k, v, num_splits=2, workspace=ws)),
        ("fwd gqa split", lambda ws: fa.fwd(q, k1, v1, num_splits=2, workspace=ws)),
        ("fwd_mxfp8 split", lambda ws: fa.fwd_mxfp8(*m8[:3], m8[3], num_splits=2, workspace=ws)),
    ]
    for name, call in calls:
        with pytest.raises(fa.FAError) as e:
            call(small)
        assert e.value.status == -9, name
        with pytest.raises(ValueError, match="workspace"):
            call(wrong)
    o, lse = fa.fwd(q, k, v, num_splits=1)
    do = torch.ones_like(q)
    bneed = fa.bwd_workspace_bytes(1, 2, N)
    with pytest.raises(fa.FAError) as e:
        fa.bwd(q, k, v, o, lse, do, workspace=torch.empty(bneed - 16, dtype=torch.uint8, device="cuda"))
    assert e.value.status == -9
    with pytest.raises(ValueError, match="workspace"):
        fa.bwd(q, k, v, o, lse, do, workspace=torch.empty(bneed, dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()


def test_caller_outputs_are_checked():
    """Outputs a caller passes in must have exactly the dtype and shape the
    kernels write (contiguous, on the device): a wrong one is refused by the
    binding before any launch."""
    print("[case] caller outputs of the wrong dtype / shape", flush=True)
    x = torch.ones((1, 2, 64, 128), dtype=torch.bfloat16, device="cuda")
    u8_short = torch.empty((1, 2, 63, 128), dtype=torch.uint8, device="cuda")
    f32_short = torch.empty(1, dtype=torch.float32, device="cuda")
    signs = torch.ones(128, dtype=torch.int8, device="cuda")
    bad = [
        lambda: fa.quantize_fp8(x, out=u8_short),
        lambda: fa.quantize_fp8(x, descale=f32_short),
        lambda: fa.quantize_fp8_rotated(x, signs, False, out=u8_short),
        lambda: fa.quantize_fp8_rotated(x, signs, False, descale=torch.empty(2, dtype=torch.float64, device="cuda")),
        lambda: fa.quantize_mxfp8_rows(x, scales=torch.empty((1, 2, 64, 2), dtype=torch.uint8, device="cuda")),
        lambda: fa.quantize_mxfp8_keys(x, scales=torch.empty((1, 2, 64, 128), dtype=torch.uint8, device="cuda")),
        lambda: fa.merge_partials(torch.zeros((2, 2, 64, 128), device="cuda"), torch.zeros((2, 2, 64), device="cuda"),
                                  out=torch.empty((2, 64, 128), dtype=torch.float32, device="cuda")),
        lambda: fa.merge_partials(torch.zeros((2, 2, 64, 128), device="cuda"), torch.zeros((2, 2, 64), device="cuda"),
                                  lse=torch.empty((2, 63), dtype=torch.float32, device="cuda")),
    ]
    for i, call in enumerate(bad):
        with pytest.raises(ValueError):
            call()
    o, lse = fa.fwd(x, x, x)
    with pytest.raises(ValueError, match="dk"):
        fa.bwd(x, x, x, o, lse, x, dk=torch.empty((1, 2, 64, 128), dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()


@pytest.mark.parametrize("H,N,causal,expect", [(4, 4096, False, 4), (8, 4096, False, 2), (32, 1024, False, 1),
                                               (8, 4096, True, 3)])
def test_default_split_matches_oracle(H, N, causal, expect):
    """fwd() with the library's own number of key chunks (fa_splitkv_default_splits
    on a 256-CU device: about two workgroups per CU, three if causal, no chunk
    under 1024 keys) against the oracle on sampled rows of every head."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    S = fa.default_splits(1, H, N, 128, causal, fa.DTYPE_BF16)
    print(f"[case] default split H={H} N={N} causal={causal}: {S} chunks on {cus} CUs", flush=True)
    if cus == 256:
        assert S == expect
    q, k, v = make_qkv(1, H, N, 128, "bf16", seed=H + N)
    o, lse = fa.fwd(q.cuda(), k.cuda(), v.cuda(), causal=causal)
    torch.cuda.synchronize()
    rows = sample_rows(N, tile=128, n_random=16)
    O_ref, L_ref = oracle.attention(q, k, v, scale=128 ** -0.5, causal=causal, rows=rows)
    got_o = o.float().cpu().double().numpy()[:, :, rows]
    got_l = lse.cpu().double().numpy()[:, :, rows]
    floor = float(np.max(np.abs(torch.from_numpy(O_ref).to(torch.bfloat16).double().numpy() - O_ref)))
    err_o, err_l = float(np.max(np.abs(got_o - O_ref))), float(np.max(np.abs(got_l - L_ref)))
    print(f"    max|dO|={err_o:.3e} (tol {1e-2 + floor:.3e}) max|dL|={err_l:.3e}", flush=True)
    assert err_o <= 1e-2 + floor and err_l <= 1e-3
