"""Pins for the split-KV oracle (CPU only): key-range partials and their merge.

"Kernels and Memory in LLM Inference", section "Flash-Decoding: one token,
whole chip": attention over contiguous key chunks, each with its own max and
sum, merged by rescaling to the overall max, is exact attention. The pins tie
attention_keyrange() and merge_partials() to things other than themselves:
the full-sequence definition (a different function), pure-Python brute force,
closed forms of one-key chunks and of equal-weight halves, and scipy's
logsumexp. Planted mistakes in copies of both functions must fail a pin.
"""
import math

import numpy as np
import pytest
from scipy.special import logsumexp

import oracle


def _rand(B, H, N, d, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, H, N, d)), rng.standard_normal((B, H, N, d)),
            rng.standard_normal((B, H, N, d)))


def _partition(N, cuts):
    edges = [0] + sorted(cuts) + [N]
    return list(zip(edges[:-1], edges[1:]))


def _split_and_merge(keyrange, merge, q, k, v, scale, causal, ranges):
    parts = [keyrange(q, k, v, scale, causal, a, b) for a, b in ranges]
    return merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))


PARTITIONS = [
    [],                       # one chunk = the whole sequence
    [37],                     # two uneven chunks
    [0, 37],                  # an empty first chunk
    [5, 5, 90],               # an empty middle chunk
    [1, 2, 3, 64, 128],       # one-key chunks and a 128-aligned cut
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("cuts", PARTITIONS)
def test_merge_of_chunks_is_full_attention(causal, cuts):
    q, k, v = _rand(1, 2, 150, 16, seed=1)
    O_ref, L_ref = oracle.attention(q, k, v, 0.3, causal=causal)
    O, L = _split_and_merge(oracle.attention_keyrange, oracle.merge_partials, q, k, v, 0.3, causal,
                            _partition(150, cuts))
    assert np.allclose(O, O_ref, atol=1e-12, rtol=0)
    assert np.allclose(L, L_ref, atol=1e-12, rtol=0)


def test_full_range_is_the_definition():
    q, k, v = _rand(2, 1, 77, 8, seed=2)
    for causal in (False, True):
        O, L = oracle.attention_keyrange(q, k, v, 0.5, causal, 0, 77)
        O_ref, L_ref = oracle.attention(q, k, v, 0.5, causal=causal)
        assert np.allclose(O, O_ref, atol=1e-13, rtol=0) and np.allclose(L, L_ref, atol=1e-13, rtol=0)


def test_bruteforce_agrees_after_merge():
    q, k, v = _rand(1, 1, 9, 3, seed=3)
    for causal in (False, True):
        O_bf, L_bf = oracle.attention_bruteforce(q, k, v, 0.7, causal=causal)
        O, L = _split_and_merge(oracle.attention_keyrange, oracle.merge_partials, q, k, v, 0.7, causal,
                                _partition(9, [2, 4, 8]))
        assert np.allclose(O, O_bf, atol=1e-13) and np.allclose(L, L_bf, atol=1e-13)


def test_one_key_chunk_closed_form():
    q, k, v = _rand(1, 1, 12, 4, seed=4)
    j = 7
    O, L = oracle.attention_keyrange(q, k, v, 0.25, False, j, j + 1)
    # softmax over one key: weight 1, L = that key's scaled score
    assert np.allclose(O[0, 0], np.broadcast_to(v[0, 0, j], (12, 4)), atol=0)
    assert np.allclose(L[0, 0], 0.25 * (q[0, 0] @ k[0, 0, j]), atol=1e-14)
    # causal: rows above key j have no valid key in the chunk
    O, L = oracle.attention_keyrange(q, k, v, 0.25, True, j, j + 1)
    assert np.all(O[0, 0, :j] == 0) and np.all(L[0, 0, :j] == -np.inf)
    assert np.allclose(O[0, 0, j:], np.broadcast_to(v[0, 0, j], (12 - j, 4)), atol=0)


def test_empty_and_out_of_range_chunks():
    q, k, v = _rand(1, 1, 10, 4, seed=5)
    for a, b in [(4, 4), (10, 20), (12, 15)]:
        O, L = oracle.attention_keyrange(q, k, v, 1.0, False, a, b)
        assert np.all(O == 0) and np.all(L == -np.inf)
    # a chunk running past N is clipped to N
    O1, L1 = oracle.attention_keyrange(q, k, v, 1.0, False, 6, 100)
    O2, L2 = oracle.attention_keyrange(q, k, v, 1.0, False, 6, 10)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


def test_merge_closed_forms():
    rng = np.random.default_rng(6)
    O1, O2 = rng.standard_normal((2, 5, 8))
    L = rng.standard_normal(5)
    # equal weights: the mean, and L + log 2
    O, Lm = oracle.merge_partials(np.stack([O1, O2]), np.stack([L, L]))
    assert np.allclose(O, 0.5 * (O1 + O2), atol=1e-15) and np.allclose(Lm, L + math.log(2), atol=1e-15)
    # weights 1 : e (L differs by exactly 1)
    O, Lm = oracle.merge_partials(np.stack([O1, O2]), np.stack([L, L + 1]))
    assert np.allclose(O, (O1 + math.e * O2) / (1 + math.e), atol=1e-14)
    # an empty chunk is ignored; every chunk empty -> O = 0, L = -inf
    ninf = np.full(5, -np.inf)
    O, Lm = oracle.merge_partials(np.stack([O1, np.zeros_like(O2)]), np.stack([L, ninf]))
    assert np.array_equal(O, O1) and np.array_equal(Lm, L)
    O, Lm = oracle.merge_partials(np.zeros((3, 5, 8)), np.stack([ninf] * 3))
    assert np.all(O == 0) and np.all(Lm == -np.inf)


def test_merge_lse_matches_scipy():
    rng = np.random.default_rng(7)
    Ls = rng.standard_normal((4, 3, 50)) * 20
    Ls[1, 0, :10] = -np.inf
    Os = rng.standard_normal((4, 3, 50, 6))
    O, L = oracle.merge_partials(Os, Ls)
    assert np.allclose(L, logsumexp(Ls, axis=0), atol=1e-12)
    w = np.exp(Ls - logsumexp(Ls, axis=0)[None])
    assert np.allclose(O, np.einsum("spr,sprd->prd", w, Os), atol=1e-12)


def test_merge_is_order_independent_and_large_l_safe():
    rng = np.random.default_rng(8)
    Ls = rng.standard_normal((5, 40)) * 1e3       # exp(L) alone would overflow
    Os = rng.standard_normal((5, 40, 4))
    O, L = oracle.merge_partials(Os, Ls)
    perm = rng.permutation(5)
    O2, L2 = oracle.merge_partials(Os[perm], Ls[perm])
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(L))
    assert np.allclose(O, O2, atol=1e-12) and np.allclose(L, L2, atol=1e-9)


# --------------------------------------------------------------------------
# planted mistakes
# --------------------------------------------------------------------------
def _keyrange_mutant(kind):
    def f(q, k, v, scale, causal, k0, k1, rows=None):
        if kind == "inclusive_end":
            k1 = k1 + 1
        if kind == "ignore_causal":
            causal = False
        O, L = oracle.attention_keyrange(q, k, v, scale, causal, k0, k1, rows)
        if kind == "l_without_log":
            L = np.exp(L)
        return O, L
    return f


def _merge_mutant(kind):
    def f(Os, Ls):
        Os = np.asarray(Os, dtype=np.float64)
        Ls = np.asarray(Ls, dtype=np.float64)
        M = Ls.max(0)
        w = np.exp(Ls - M[None])
        if kind == "unweighted":
            w = np.ones_like(w)
        if kind == "unnormalised":
            return (w[..., None] * Os).sum(0), M + np.log(w.sum(0))
        if kind == "lse_is_max":
            return (w[..., None] * Os).sum(0) / w.sum(0)[..., None], M
        if kind == "weights_from_max_only":
            w = (Ls == M[None]).astype(np.float64)
        return (w[..., None] * Os).sum(0) / w.sum(0)[..., None], M + np.log(w.sum(0))
    return f


def _pins_pass(keyrange, merge) -> bool:
    try:
        q, k, v = _rand(1, 2, 60, 8, seed=9)
        for causal in (False, True):
            O_ref, L_ref = oracle.attention(q, k, v, 0.3, causal=causal)
            O, L = _split_and_merge(keyrange, merge, q, k, v, 0.3, causal, _partition(60, [13, 31, 32]))
            if not (np.allclose(O, O_ref, atol=1e-10) and np.allclose(L, L_ref, atol=1e-10)):
                return False
        return True
    except Exception:
        return False


def test_pins_accept_the_oracle():
    assert _pins_pass(oracle.attention_keyrange, oracle.merge_partials)


@pytest.mark.parametrize("kind", ["inclusive_end", "ignore_causal", "l_without_log"])
def test_pins_reject_keyrange_mistake(kind):
    assert not _pins_pass(_keyrange_mutant(kind), oracle.merge_partials)


@pytest.mark.parametrize("kind", ["unweighted", "unnormalised", "lse_is_max", "weights_from_max_only"])
def test_pins_reject_merge_mistake(kind):
    assert not _pins_pass(oracle.attention_keyrange, _merge_mutant(kind))
