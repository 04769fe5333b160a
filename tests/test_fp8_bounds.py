"""The per-element FP8 bounds (tests/fp8_bounds.py) against a CPU emulation
of the kernel's P arithmetic.

The emulation follows the FP8 forward's recipe in float64 ("1.8x Faster
Attention on an RTX 5080", sections "The loop starts" through "After the last
strip" and "P goes through shared memory, then P.V"; "Kernels and Memory in
LLM Inference", section "FlashAttention-4" for the lagging reference): keys in
tiles of 64; a reference max that moves only when a tile's max exceeds it by
more than tau = 0.75 (log2 units), exactly then, for every row of the
32-row group the tile is processed for (as a wave does); p = 2^(s c - m_ref);
l sums the unrounded p; O sums e4m3(256 p) v, divided by 256 l; L = ln 2
(m_ref + log2 l). The only rounding it models is P's, so its distance to the
oracle must sit inside the P-rounding part of the bounds (no MFMA error:
eps_acc = 0) on every element, and the bounds must not be vacuous: somewhere
the emulated error reaches a sizeable share of them.
"""
import math

import numpy as np
import pytest

import oracle
from fp8_bounds import fp8_bounds
from tiled_attention_fa2_amd.inputs import make_qkv

LOG2E = 1.4426950408889634


def _emulate(q, k, v, scale, causal, tau=0.75, bn=64, rows_per_wave=32):
    """float64 emulation of the FP8 kernel's softmax and P rounding on
    dequantised inputs [B, H, N, d]; returns (O, L)."""
    B, H, N, d = q.shape
    O = np.zeros((B, H, N, d))
    L = np.zeros((B, H, N))
    c = scale * LOG2E
    for b in range(B):
        for h in range(H):
            T = (q[b, h] @ k[b, h].T) * c                     # log2-domain scores
            if causal:
                T = np.where(np.arange(N)[None, :] <= np.arange(N)[:, None], T, -np.inf)
            for w0 in range(0, N, rows_per_wave):
                rows = np.arange(w0, min(N, w0 + rows_per_wave))
                m_ref = np.full(len(rows), -np.inf)
                l = np.zeros(len(rows))
                acc = np.zeros((len(rows), d))
                for j0 in range(0, N, bn):
                    t = T[rows, j0:j0 + bn]
                    if causal and j0 > rows[-1]:
                        break
                    ext = np.max(t, axis=1)
                    if np.any(ext > m_ref + tau):
                        m_new = np.maximum(m_ref, ext)
                        alpha = np.exp2(m_ref - m_new)
                        m_ref = m_new
                        l *= alpha
                        acc *= alpha[:, None]
                    p = np.exp2(t - m_ref[:, None])
                    l += p.sum(axis=1)
                    pr = oracle.e4m3_decode(oracle.e4m3_encode(256.0 * p)) / 256.0
                    acc += pr @ v[b, h, j0:j0 + bn]
                O[b, h, rows] = acc / l[:, None]
                L[b, h, rows] = (m_ref + np.log2(l)) / LOG2E
    return O, L


def _dequantised(variant, N, seed):
    q, k, v = make_qkv(1, 2, N, 128, "bf16", seed=seed, variant=variant)
    return tuple(oracle.dequantize_per_head(*oracle.quantize_per_head(t)) for t in (q, k, v))


@pytest.mark.parametrize("variant", ["iid", "peaked", "growing", "outlier"])
@pytest.mark.parametrize("causal", [False, True])
def test_bounds_hold_for_the_emulated_p_rounding(variant, causal):
    N = 300
    scale = 1.0 / math.sqrt(128)
    ref_in = _dequantised(variant, N, seed=11)
    O_ref, L_ref = oracle.attention(*ref_in, scale=scale, causal=causal)
    O_em, L_em = _emulate(*ref_in, scale, causal)
    bO, bL, nv = fp8_bounds(ref_in, scale, L_ref, O_ref, causal=causal, eps_acc=0.0)
    ratio = np.abs(O_em - O_ref) / bO
    print(f"{variant} causal={causal}: max|dO| {np.abs(O_em - O_ref).max():.3e}, "
          f"max dO/bound {ratio.max():.3f}, max|dL| {np.abs(L_em - L_ref).max():.3e}")
    assert ratio.max() <= 1.0
    # L: the emulation sums unrounded p in float64, so L is exact up to float64
    assert np.abs(L_em - L_ref).max() <= 1e-9
    # not vacuous: the rounding uses a real share of the bound somewhere
    assert ratio.max() >= 0.05


def test_bound_reaches_the_worst_case_on_a_one_hot_row():
    # one key far above the rest: the row's weight is that key's alone, and
    # with a reference that lags (the key's weight 1.56 against the earlier max)
    # its e4m3 rounding is the whole error, which the worst-case term bounds
    N, d = 128, 128
    rng = np.random.default_rng(3)
    q = np.zeros((1, 1, N, d))
    k = rng.standard_normal((1, 1, N, d)) * 0.01
    v = rng.standard_normal((1, 1, N, d))
    q[0, 0, :, 0] = 1.0
    k[0, 0, 10, 0] = 10.0                      # max of tile 0
    k[0, 0, 70, 0] = 10.0 + math.log2(1.56) / LOG2E   # tile 1: p = 1.56 (< 2^tau), 256 p rounds 4% off
    scale = 1.0
    O_ref, L_ref = oracle.attention(q, k, v, scale=scale)
    O_em, _ = _emulate(q, k, v, scale, causal=False)
    bO, _, _ = fp8_bounds((q, k, v), scale, L_ref, O_ref, eps_acc=0.0)
    ratio = np.abs(O_em - O_ref) / bO
    assert ratio.max() <= 1.0
    assert ratio.max() >= 0.1


def test_planted_mistake_in_the_bound_is_caught():
    # a bound that forgets the e4m3 rounding of P (only the MFMA term left)
    # must fail on the emulated errors
    N = 200
    scale = 1.0 / math.sqrt(128)
    ref_in = _dequantised("peaked", N, seed=5)
    O_ref, L_ref = oracle.attention(*ref_in, scale=scale)
    O_em, _ = _emulate(*ref_in, scale, causal=False)
    bO, _, _ = fp8_bounds(ref_in, scale, L_ref, O_ref, eps_acc=0.0)
    import fp8_bounds as fb

    saved = fb.EPS_E4M3, fb.SIGMA_E4M3
    try:
        fb.EPS_E4M3, fb.SIGMA_E4M3 = 0.0, 0.0
        bO_bad, _, _ = fp8_bounds(ref_in, scale, L_ref, O_ref, eps_acc=0.0)
    finally:
        fb.EPS_E4M3, fb.SIGMA_E4M3 = saved
    assert (np.abs(O_em - O_ref) / bO).max() <= 1.0
    assert (np.abs(O_em - O_ref) / bO_bad).max() > 1.0


def _round_bf16(x):
    """Round float64 values to bf16 (round to nearest, ties to even) through
    float32, as the kernel's v_cvt_pk_bf16_f32 does with fp32 p."""
    import torch
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).double().numpy()


def _emulate_bf16(q, k, v, scale, causal):
    """float64 emulation of the bf16 kernel's P rounding: exact running max,
    p = 2^(s c - m) (the largest weight exactly 1), l over unrounded p, O over
    bf16-rounded p. The reference max is the row's final max: rescales by
    alpha = 2^(m_old - m_new) are applied to the rounded p of earlier tiles in
    fp32 by the kernel, which does not change their relative error."""
    B, H, N, d = q.shape
    O = np.zeros((B, H, N, d))
    c = scale * LOG2E
    for b in range(B):
        for h in range(H):
            T = (q[b, h] @ k[b, h].T) * c
            if causal:
                T = np.where(np.arange(N)[None, :] <= np.arange(N)[:, None], T, -np.inf)
            m = np.max(T, axis=1, keepdims=True)
            p = np.exp2(T - m)
            O[b, h] = (_round_bf16(p) @ v[b, h]) / p.sum(axis=1, keepdims=True)
    return O


@pytest.mark.parametrize("variant", ["outlier", "peaked"])
def test_bf16_p_rounding_bound_holds_and_is_not_vacuous(variant):
    # the bf16 stress tolerance term 2^-8 sum_j P_ij |v_jd| of the parity tests
    from fp8_bounds import p_weighted_abs_v
    q, k, v = (t.double().numpy() for t in make_qkv(1, 2, 257, 64, "bf16", seed=5, variant=variant))
    scale = 1.0 / math.sqrt(64)
    for causal in (False, True):
        O_ref, L_ref = oracle.attention(q, k, v, scale=scale, causal=causal)
        O_em = _emulate_bf16(q, k, v, scale, causal)
        bound = 2.0 ** -8 * p_weighted_abs_v((q, k, v), scale, L_ref, causal=causal)
        ratio = np.abs(O_em - O_ref) / np.maximum(bound, 1e-300)
        assert ratio.max() <= 1.0, (variant, causal, ratio.max())
        assert ratio.max() >= 0.05, (variant, causal, ratio.max())
