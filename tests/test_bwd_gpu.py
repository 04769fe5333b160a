"""Parity of the HIP backward (fa_bwd, through the C ABI) with the fp64 oracle.

The forward runs on the GPU first (its bf16 O and fp32 L are the backward's
inputs, as in training); the oracle gets the same Q, K, V, dO and the same O
(D = rowsum(dO * O) is formed from the O the caller holds) and computes
dQ, dK, dV exactly. Tolerance per tensor (max-abs over all elements), from the
arithmetic: the products take P and dS rounded to bf16 (relative 2^-9 each)
and the outputs are bf16, so an error of a few 2^-9 of the tensor's largest
magnitude plus the bf16 rounding floor of the exact answer; the test uses
1e-2 * max|ref| + that floor, and cosine >= 0.9999.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from tiled_attention_fa2_amd import fa
from tiled_attention_fa2_amd.inputs import make_dout, make_gqa, make_qkv

pytestmark = pytest.mark.gpu


def _floor(ref):
    return float(np.max(np.abs(torch.from_numpy(ref).to(torch.bfloat16).double().numpy() - ref)))


def _cos(a, b):
    a, b = a.ravel(), b.ravel()
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b) + 1e-300))


def _check(q, k, v, do, causal, scale, label):
    print(f"[case] {label} q={tuple(q.shape)} k={tuple(k.shape)} causal={causal} scale={scale}", flush=True)
    qd, kd, vd, dod = (t.cuda().contiguous() for t in (q, k, v, do))
    o, lse = fa.fwd(qd, kd, vd, causal=causal, scale=scale, num_splits=1)
    dq, dk, dv = fa.bwd(qd, kd, vd, o, lse, dod, causal=causal, scale=scale)
    torch.cuda.synchronize()
    group = q.shape[1] // k.shape[1]
    kr = k.repeat_interleave(group, dim=1)
    vr = v.repeat_interleave(group, dim=1)
    dQ, dKr, dVr, _ = oracle.attention_backward(q, kr, vr, do, scale, causal=causal, o=o.cpu())
    B, Hkv, N, d = k.shape
    dK = dKr.reshape(B, Hkv, group, N, d).sum(axis=2)   # a shared K/V head sums its group's gradients
    dV = dVr.reshape(B, Hkv, group, N, d).sum(axis=2)
    for name, got, ref in (("dq", dq, dQ), ("dk", dk, dK), ("dv", dv, dV)):
        g = got.float().cpu().double().numpy()
        err = float(np.max(np.abs(g - ref)))
        tol = 1e-2 * float(np.max(np.abs(ref))) + _floor(ref)
        cos = _cos(g, ref)
        print(f"    {name}: max|err|={err:.3e} tol={tol:.3e} max|ref|={np.max(np.abs(ref)):.3e} cos={cos:.7f}",
              flush=True)
        assert np.all(np.isfinite(g)), name
        assert err <= tol, (label, name, err, tol)
        if np.any(ref):
            assert cos >= 0.9999, (label, name, cos)
        else:   # an exactly zero gradient (one key: dS = 0) must come out exactly zero
            assert not np.any(g), (label, name)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_oracle(d, causal):
    for B, H, N in [(1, 2, 300), (2, 1, 129), (1, 1, 1), (1, 2, 777)]:
        q, k, v = make_qkv(B, H, N, d, "bf16", seed=N + d)
        do = make_dout(B, H, N, d, seed=N + d + 1)
        _check(q, k, v, do, causal, 1.0 / math.sqrt(d), label=f"N={N} d={d}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_dq_key_split(d, causal):
    # grids too small for two dQ workgroups per CU cut the keys into chunks of
    # >= 1024 whose partial dQ are summed in order: 2 x 2500 tokens takes 2
    # chunks, 2 x 3333 (ragged) 3 on a 256-CU device
    for B, H, N in [(1, 2, 2500), (1, 2, 3333)]:
        assert fa.bwd_workspace_bytes(B, H, N) > 8 * B * H * N, "the key split is not taken"
        q, k, v = make_qkv(B, H, N, d, "bf16", seed=N + d + 5)
        do = make_dout(B, H, N, d, seed=N + d + 6)
        _check(q, k, v, do, causal, 1.0 / math.sqrt(d), label=f"dQ key split N={N} d={d}")
    # deterministic: the partials are summed in chunk order
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    o, lse = fa.fwd(qd, kd, vd, causal=causal, num_splits=1)
    a = fa.bwd(qd, kd, vd, o, lse, dod, causal=causal)
    b = fa.bwd(qd, kd, vd, o, lse, dod, causal=causal)
    torch.cuda.synchronize()
    assert all(torch.equal(x.view(torch.int16), y.view(torch.int16)) for x, y in zip(a, b))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_gqa(d, causal):
    q, k, v = make_gqa(1, 8, 2, 400, d, "bf16", seed=3)
    do = make_dout(1, 8, 400, d, seed=4)
    _check(q, k, v, do, causal, 1.0 / math.sqrt(d), label=f"gqa 8/2 d={d}")


@pytest.mark.parametrize("scale", [0.0, -0.09, 0.3])
def test_backward_scale_values(scale):
    q, k, v = make_qkv(1, 2, 260, 64, "bf16", seed=5)
    do = make_dout(1, 2, 260, 64, seed=6)
    for causal in (False, True):
        _check(q, k, v, do, causal, scale, label=f"scale={scale}")


def test_backward_stress_inputs():
    for variant in ("peaked", "growing"):
        q, k, v = make_qkv(1, 2, 512, 128, "bf16", seed=7, variant=variant)
        do = make_dout(1, 2, 512, 128, seed=8)
        for causal in (False, True):
            _check(q, k, v, do, causal, 1.0 / math.sqrt(128), label=variant)


def test_backward_masked_scores_overflow():
    """Causal rows whose masked (future) keys score far above their own
    logsumexp: the last 16 keys of the sequence have norms 60x the others, so
    for the earlier queries exp2(S c - L2) of those masked slots overflows in
    float32 (checked below on the CPU). The dK/dV kernel computes masked slots
    like the others and zeroes them afterwards; the gradients must stay finite
    and match the oracle."""
    N, d = 300, 128
    q, k, v = make_qkv(1, 2, N, d, "bf16", seed=11)
    k = k.clone()
    k[:, :, N - 16:, :] = (k[:, :, N - 16:, :].float() * 60.0).to(torch.bfloat16)
    do = make_dout(1, 2, N, d, seed=12)
    scale = 1.0 / math.sqrt(d)
    # the overflow happens where the kernel computes masked slots (queries of
    # the last 64 rows, the diagonal tiles of the last keys): some masked
    # (query, key) pair has S c - L2 > 128
    _, L = oracle.attention(q, k, v, scale, causal=True)
    S = np.einsum("bhqd,bhkd->bhqk", q.double().numpy(), k.double().numpy()) * scale
    excess = (S - L[..., None]) * math.log2(math.e)
    future = np.triu(np.ones((N, N), dtype=bool), 1)[N - 64:, N - 16:]
    assert np.max(excess[:, :, N - 64:, N - 16:][..., future]) > 130.0
    _check(q, k, v, do, True, scale, label="masked overflow")


def test_backward_deterministic():
    q, k, v = (t.cuda() for t in make_qkv(1, 4, 1000, 128, "bf16", seed=9))
    do = make_dout(1, 4, 1000, 128, seed=10).cuda()
    o, lse = fa.fwd(q, k, v, causal=True, num_splits=1)
    a = fa.bwd(q, k, v, o, lse, do, causal=True)
    b = fa.bwd(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(a, b))


def test_backward_rejects_bad_arguments():
    q, k, v = (t.cuda() for t in make_qkv(1, 1, 64, 64, "bf16", seed=1))
    o, lse = fa.fwd(q, k, v, num_splits=1)
    do = torch.zeros_like(q)
    with pytest.raises(TypeError):
        fa.bwd(q.float(), k.float(), v.float(), o, lse, do)
    small = torch.empty(8, dtype=torch.uint8, device="cuda")
    with pytest.raises(fa.FAError) as e:
        fa.bwd(q, k, v, o, lse, do, workspace=small)
    assert e.value.status == -9


def test_backward_full_size_sampled():
    # the 56-head x 30272-token DiT shape: the whole backward on the GPU,
    # heads 0 and 55 checked on sampled query rows (dQ) and key rows (dK, dV)
    from tiled_attention_fa2_amd.inputs import WORKLOADS, sample_rows
    w = WORKLOADS["bf16_dit_b1_h56_n30272_d128"]
    q, k, v = make_qkv(w.B, w.H, w.N, w.d, "bf16", seed=0)
    do = make_dout(w.B, w.H, w.N, w.d, seed=1)
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    print(f"[case] full-size backward {w.name}", flush=True)
    o, lse = fa.fwd(qd, kd, vd, scale=w.scale, num_splits=1)
    dq, dk, dv = fa.bwd(qd, kd, vd, o, lse, dod, scale=w.scale)
    torch.cuda.synchronize()
    q_rows = sample_rows(w.N, tile=128, n_random=16)
    k_rows = sample_rows(w.N, tile=128, n_random=16, seed=54321)
    heads = [(0, 0), (0, 55)]
    rq, rk, rv = oracle.attention_backward_rows(q, k, v, do, w.scale, False, o.cpu(), q_rows, k_rows,
                                                heads=heads)
    for t, (b, h) in enumerate(heads):
        for name, got, ref in (("dq", dq[b, h, q_rows], rq[t]), ("dk", dk[b, h, k_rows], rk[t]),
                               ("dv", dv[b, h, k_rows], rv[t])):
            g = got.float().cpu().double().numpy()
            err = float(np.max(np.abs(g - ref)))
            tol = 1e-2 * float(np.max(np.abs(ref))) + _floor(ref)
            print(f"    head {h} {name}: max|err|={err:.3e} tol={tol:.3e} cos={_cos(g, ref):.7f}", flush=True)
            assert err <= tol and _cos(g, ref) >= 0.9999, (h, name)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_key_blocks_per_wave(d, causal):
    """The dK/dV kernel runs two 32-key blocks per wave when B*Hkv*ceil(N/256)
    fills the device's compute units, else one (twice the workgroups). 128
    heads of 512 tokens take two blocks on a 256-CU device; any one head alone
    takes one. The gradients of a head must be identical either way (the
    blocks change which workgroup owns a key, never the arithmetic of its
    gradient), and sampled heads of the 128-head launch must match the oracle."""
    B, H, N = 1, 128, 512
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert B * H * -(-N // 256) >= cus, "shape no longer selects two blocks per wave on this device"
    print(f"[case] key blocks per wave d={d} causal={causal} H={H} N={N} cus={cus}", flush=True)
    scale = 1.0 / math.sqrt(d)
    q, k, v = (t.cuda().contiguous() for t in make_qkv(B, H, N, d, "bf16", seed=61))
    do = make_dout(B, H, N, d, seed=62).cuda().contiguous()
    o, lse = fa.fwd(q, k, v, causal=causal, scale=scale, num_splits=1)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=causal, scale=scale)
    torch.cuda.synchronize()
    for h in (0, 77, H - 1):
        one = [t[:, h:h + 1].contiguous() for t in (q, k, v, o, lse, do)]
        g1 = fa.bwd(*one, causal=causal, scale=scale)
        torch.cuda.synchronize()
        for name, got, full in zip(("dq", "dk", "dv"), g1, (dq, dk, dv)):
            assert torch.equal(got, full[:, h:h + 1]), (h, name)
    for h in (0, H - 1):
        sl = [t[:, h:h + 1].cpu() for t in (q, k, v, do)]
        dQ, dK, dV, _ = oracle.attention_backward(*sl, scale, causal=causal, o=o[:, h:h + 1].cpu())
        for name, got, ref in (("dq", dq, dQ), ("dk", dk, dK), ("dv", dv, dV)):
            g = got[:, h:h + 1].float().cpu().double().numpy()
            err = float(np.max(np.abs(g - ref)))
            tol = 1e-2 * float(np.max(np.abs(ref))) + _floor(ref)
            print(f"    head {h} {name}: max|err|={err:.3e} tol={tol:.3e} cos={_cos(g, ref):.7f}", flush=True)
            assert np.all(np.isfinite(g)) and err <= tol and _cos(g, ref) >= 0.9999, (h, name)
