"""Pins for the fp64 attention oracle (CPU only).

Each check ties the oracle to something other than itself: a worked example
the pages print, closed forms of the softmax, an independent library routine,
a second (tiled, online) formulation, pure-Python brute force, and invariants.
A final group plants plausible mistakes in copies of the oracle and checks
that at least one pin catches each of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle
from tiled_attention_fa2_amd.inputs import make_qkv, sample_rows

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(B, H, N, d, seed=0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, H, N, d)), rng.standard_normal((B, H, N, d)),
            rng.standard_normal((B, H, N, d)))


# --------------------------------------------------------------------------
# worked example printed on "1.8x Faster Attention on an RTX 5080"
# --------------------------------------------------------------------------
def _worked_example_inputs():
    ex = json.load(open(os.path.join(GOLDEN, "worked_example_online_softmax.json")))
    scores = [s for strip in ex["scores_by_strip"] for s in strip]
    n = len(scores)
    # q = e0 and k_j = scores[j] * e0 with scale 1 make S = scores; V = I makes O = weights
    d = n
    q = np.zeros((1, 1, n, d))
    q[0, 0, :, 0] = 1.0
    k = np.zeros((1, 1, n, d))
    k[0, 0, :, 0] = scores
    v = np.eye(n).reshape(1, 1, n, d)
    return ex, q, k, v


def test_worked_example_online_trace():
    ex, q, k, v = _worked_example_inputs()
    tol = 0.5 * 10 ** (-ex["printed_decimals"])
    O, L, tr = oracle.attention_online(q, k, v, scale=1.0, tile_q=4, tile_k=2, trace=True)
    steps = tr[(0, 0, 0)]
    assert len(steps) == 2
    (m0, l0, _), (m1, l1, a1) = steps
    assert m0 == ex["m_after_strip"][0] and m1 == ex["m_after_strip"][1]
    assert abs(l0 - ex["l_after_strip"][0]) <= tol
    assert abs(a1 - ex["alpha_strip1"]) <= tol
    assert abs(l1 - ex["l_after_strip"][1]) <= tol
    # unnormalised weights e^(s - m_final): l times the normalised ones
    unnorm = O[0, 0, 0] * l1
    assert np.allclose(unnorm, ex["unnormalised_weights"], atol=0.5 * 10 ** (-ex["unnormalised_weights_decimals"]))


def test_worked_example_definition():
    ex, q, k, v = _worked_example_inputs()
    tol = 0.5 * 10 ** (-ex["printed_decimals"])
    O, L = oracle.attention(q, k, v, scale=1.0)
    assert np.allclose(O[0, 0, 0], ex["weights"], atol=tol)
    # L = m + log(l) with the page's l over all keys at once
    assert abs(L[0, 0, 0] - (ex["m_after_strip"][1] + math.log(ex["l_all_keys_at_once"]))) <= 1e-3


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
def test_rows_sum_to_one_identity_v(causal):
    # V = I_N (d = N) turns O into the probability matrix P itself
    N = 13
    rng = np.random.default_rng(1)
    q = rng.standard_normal((1, 2, N, N))
    k = rng.standard_normal((1, 2, N, N))
    v = np.broadcast_to(np.eye(N), (1, 2, N, N)).copy()
    O, L = oracle.attention(q, k, v, scale=0.3, causal=causal)
    assert np.all(O >= 0)
    assert np.allclose(O.sum(-1), 1.0, atol=1e-12)
    if causal:
        assert np.all(np.triu(O[0, 0], 1) == 0)
    # P_ij = exp(S_ij - L_i) entry by entry (catches a transposed K or V)
    S = 0.3 * q[0, 1] @ k[0, 1].T
    P = np.exp(S - L[0, 1][:, None])
    if causal:
        P = np.tril(P)
    assert np.allclose(O[0, 1], P, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_identical_keys_give_mean_of_v(causal):
    N, d = 17, 8
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 1, N, d))
    k = np.broadcast_to(rng.standard_normal(d), (1, 1, N, d)).copy()
    v = rng.standard_normal((1, 1, N, d))
    scale = 0.7
    O, L = oracle.attention(q, k, v, scale, causal=causal)
    for i in range(N):
        n_valid = i + 1 if causal else N
        assert np.allclose(O[0, 0, i], v[0, 0, :n_valid].mean(0), atol=1e-12)
        s = scale * q[0, 0, i] @ k[0, 0, 0]
        assert abs(L[0, 0, i] - (s + math.log(n_valid))) < 1e-12


def test_constant_v_rows():
    q, k, _ = _rand(1, 2, 21, 16, seed=3)
    c = np.linspace(-2, 3, 16)
    v = np.broadcast_to(c, (1, 2, 21, 16)).copy()
    for causal in (False, True):
        O, _ = oracle.attention(q, k, v, 0.25, causal=causal)
        assert np.allclose(O, c, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_lse_matches_scipy_logsumexp(causal):
    q, k, v = _rand(2, 3, 29, 16, seed=4)
    scale = 1 / 4
    _, L = oracle.attention(q, k, v, scale, causal=causal)
    for b in range(2):
        for h in range(3):
            S = scale * q[b, h] @ k[b, h].T
            if causal:
                S = np.where(np.tri(29, dtype=bool), S, -np.inf)
            assert np.allclose(L[b, h], logsumexp(S, axis=1), atol=1e-12, rtol=0)


@pytest.mark.parametrize("causal", [False, True])
def test_scale_zero(causal):
    q, k, v = _rand(1, 2, 23, 8, seed=5)
    O, L = oracle.attention(q, k, v, 0.0, causal=causal)
    for i in range(23):
        n = i + 1 if causal else 23
        assert np.allclose(O[:, :, i], v[:, :, :n].mean(2), atol=1e-12)
        assert np.allclose(L[:, :, i], math.log(n), atol=1e-12)


def test_causal_row_zero_and_single_key():
    q, k, v = _rand(2, 2, 9, 8, seed=6)
    O, L = oracle.attention(q, k, v, 0.5, causal=True)
    assert np.allclose(O[:, :, 0], v[:, :, 0], atol=1e-14)
    assert np.allclose(L[:, :, 0], 0.5 * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]), atol=1e-12)
    q1, k1, v1 = _rand(1, 3, 1, 8, seed=7)
    for causal in (False, True):
        O, L = oracle.attention(q1, k1, v1, 0.9, causal=causal)
        assert np.allclose(O, v1, atol=1e-14)
        assert np.allclose(L[..., 0], 0.9 * np.einsum("bhd,bhd->bh", q1[:, :, 0], k1[:, :, 0]), atol=1e-12)


# --------------------------------------------------------------------------
# library routine: fp64 CPU SDPA and torch.logsumexp
# --------------------------------------------------------------------------
@pytest.mark.parametrize("shape", [(2, 2, 100, 64), (1, 1, 37, 32), (1, 2, 200, 128), (1, 3, 64, 16)])
@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_sdpa_fp64(shape, causal):
    B, H, N, d = shape
    g = torch.Generator().manual_seed(0)
    q, k, v = (torch.randn(shape, generator=g, dtype=torch.float64) for _ in range(3))
    scale = 1 / math.sqrt(d)
    O_t = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal, scale=scale)
    S = (q @ k.transpose(-1, -2)) * scale
    if causal:
        S = S.masked_fill(~torch.ones(N, N, dtype=torch.bool).tril(), float("-inf"))
    L_t = torch.logsumexp(S, dim=-1)
    O, L = oracle.attention(q, k, v, scale, causal=causal)
    assert np.allclose(O, O_t.numpy(), atol=1e-12, rtol=0)
    assert np.allclose(L, L_t.numpy(), atol=1e-12, rtol=0)


# --------------------------------------------------------------------------
# brute force: the tiled online softmax and pure-Python loops
# --------------------------------------------------------------------------
@pytest.mark.parametrize("N", [1, 5, 16, 37, 64])
@pytest.mark.parametrize("causal", [False, True])
def test_online_tiled_matches_definition(N, causal):
    q, k, v = _rand(1, 2, N, 16, seed=N)
    O_ref, L_ref = oracle.attention(q, k, v, 0.3, causal=causal)
    for tq in (1, 3, 16, 64, N):
        for tk in (1, 3, 16, 64, N):
            O, L = oracle.attention_online(q, k, v, 0.3, causal=causal, tile_q=tq, tile_k=tk)
            assert np.allclose(O, O_ref, atol=1e-12, rtol=0), (tq, tk)
            assert np.allclose(L, L_ref, atol=1e-12, rtol=0), (tq, tk)


@pytest.mark.parametrize("causal", [False, True])
def test_pure_python_bruteforce(causal):
    q, k, v = _rand(1, 2, 5, 3, seed=11)
    O_ref, L_ref = oracle.attention(q, k, v, 0.8, causal=causal)
    O, L = oracle.attention_bruteforce(q, k, v, 0.8, causal=causal)
    assert np.allclose(O, O_ref, atol=1e-13) and np.allclose(L, L_ref, atol=1e-13)


# --------------------------------------------------------------------------
# invariants
# --------------------------------------------------------------------------
def test_key_value_permutation_invariance():
    q, k, v = _rand(1, 2, 50, 16, seed=12)
    perm = np.random.default_rng(0).permutation(50)
    O1, L1 = oracle.attention(q, k, v, 0.25)
    O2, L2 = oracle.attention(q, k[:, :, perm], v[:, :, perm], 0.25)
    assert np.allclose(O1, O2, atol=1e-12) and np.allclose(L1, L2, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_v_affine(causal):
    q, k, v = _rand(1, 1, 40, 8, seed=13)
    rng = np.random.default_rng(1)
    A = rng.standard_normal((8, 8))
    bvec = rng.standard_normal(8)
    O1, _ = oracle.attention(q, k, v, 0.4, causal=causal)
    O2, _ = oracle.attention(q, k, v @ A + bvec, 0.4, causal=causal)
    assert np.allclose(O2, O1 @ A + bvec, atol=1e-11)


def test_row_sampling_matches_full():
    q, k, v = (t.double().numpy() for t in make_qkv(1, 2, 300, 32, "bf16", seed=0))
    rows = sample_rows(300, tile=128, n_random=10)
    assert rows[0] == 0 and rows[-1] == 299 and 256 in rows
    for causal in (False, True):
        O, L = oracle.attention(q, k, v, 0.2, causal=causal)
        Os, Ls = oracle.attention(q, k, v, 0.2, causal=causal, rows=rows)
        assert np.array_equal(Os, O[:, :, rows]) and np.array_equal(Ls, L[:, :, rows])


# --------------------------------------------------------------------------
# planted mistakes: every mutant of the oracle must fail at least one pin
# --------------------------------------------------------------------------
def _mutant(kind):
    def f(q, k, v, scale, causal=False, rows=None):
        q = np.asarray(q, dtype=np.float64)
        k = np.asarray(k, dtype=np.float64)
        v = np.asarray(v, dtype=np.float64)
        N = q.shape[2]
        rows_ = np.arange(N) if rows is None else np.asarray(rows)
        O = np.zeros(q.shape[:2] + (len(rows_), q.shape[3]))
        L = np.zeros(q.shape[:2] + (len(rows_),))
        for b in range(q.shape[0]):
            for h in range(q.shape[1]):
                kk = k[b, h]
                sc = 1.0 if kind == "no_scale" else scale
                S = sc * (q[b, h, rows_] @ kk.T)
                if kind == "transposed_scores":
                    S = sc * (kk[rows_] @ q[b, h].T)
                if causal:
                    keep = (np.arange(N)[None, :] >= rows_[:, None]) if kind == "causal_flipped" \
                        else (np.arange(N)[None, :] <= rows_[:, None])
                    if kind == "causal_strict":
                        keep = np.arange(N)[None, :] < rows_[:, None]
                        keep[:, 0] = True
                    S = np.where(keep, S, -np.inf)
                m = S.max(1, keepdims=True)
                l = np.exp(S - m).sum(1, keepdims=True)
                Lr = (m + (np.log2(l) if kind == "log2_lse" else np.log(l)))[:, 0]
                if kind == "lse_without_max":
                    Lr = np.log(l[:, 0])
                P = np.exp(S - Lr[:, None])
                if kind == "unnormalised":
                    P = np.exp(S - m)
                vv = v[b, h]
                if kind == "v_transposed":
                    vv = vv.T if vv.shape[0] == vv.shape[1] else vv[::-1]
                O[b, h] = P @ vv
                L[b, h] = Lr
        return O, L
    return f


MUTANTS = ["no_scale", "transposed_scores", "causal_flipped", "causal_strict", "log2_lse",
           "lse_without_max", "unnormalised", "v_transposed"]


def _pins_pass(fn) -> bool:
    """Re-run the pins above against a candidate oracle; False if any fails."""
    try:
        # worked example (scale 1)
        ex, q, k, v = _worked_example_inputs()
        O, L = fn(q, k, v, 1.0)
        if not np.allclose(O[0, 0, 0], ex["weights"], atol=5e-4):
            return False
        if abs(L[0, 0, 0] - (4 + math.log(ex["l_all_keys_at_once"]))) > 1e-3:
            return False
        # SDPA fp64 (non-causal and causal), ragged shape
        for causal in (False, True):
            g = torch.Generator().manual_seed(0)
            qt, kt, vt = (torch.randn((1, 2, 37, 32), generator=g, dtype=torch.float64) for _ in range(3))
            O_t = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=causal, scale=0.2)
            S = (qt @ kt.transpose(-1, -2)) * 0.2
            if causal:
                S = S.masked_fill(~torch.ones(37, 37, dtype=torch.bool).tril(), float("-inf"))
            O, L = fn(qt.numpy(), kt.numpy(), vt.numpy(), 0.2, causal=causal)
            if not (np.allclose(O, O_t.numpy(), atol=1e-10) and np.allclose(L, torch.logsumexp(S, -1).numpy(), atol=1e-10)):
                return False
        return True
    except Exception:
        return False


def test_pins_accept_the_oracle():
    assert _pins_pass(oracle.attention)


@pytest.mark.parametrize("kind", MUTANTS)
def test_pins_reject_planted_mistake(kind):
    assert not _pins_pass(_mutant(kind)), kind
