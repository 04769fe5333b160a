"""Pins for the grouped-query attention oracle (CPU only).

"Kernels and Memory in LLM Inference", section "Store less: MQA, GQA, MLA":
groups of query heads share one key/value head; one group is MQA, one group
per head is MHA. attention_gqa() is pinned to torch's fp64 scaled-dot-product
attention with enable_gqa (an independent library routine that groups
consecutive query heads), to MHA when the group size is 1, to per-head
brute force, and to the closed form that the query heads of one group see
identical keys; planted mistakes in the head mapping must fail a pin.
"""
import numpy as np
import pytest
import torch

import oracle


def _rand(B, Hq, Hkv, N, d, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((B, Hq, N, d), generator=g, dtype=torch.float64)
    k = torch.randn((B, Hkv, N, d), generator=g, dtype=torch.float64)
    v = torch.randn((B, Hkv, N, d), generator=g, dtype=torch.float64)
    return q, k, v


def _sdpa(q, k, v, scale, causal):
    O = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal, scale=scale,
                                                         enable_gqa=True)
    group = q.shape[1] // k.shape[1]
    kk = k.repeat_interleave(group, dim=1)
    S = (q @ kk.transpose(-1, -2)) * scale
    if causal:
        N = q.shape[2]
        S = S.masked_fill(~torch.ones(N, N, dtype=torch.bool).tril(), float("-inf"))
    return O.numpy(), torch.logsumexp(S, -1).numpy()


@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (6, 1), (4, 4), (12, 3)])
@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_sdpa_with_gqa(Hq, Hkv, causal):
    q, k, v = _rand(2, Hq, Hkv, 37, 16, seed=Hq * 10 + Hkv)
    O, L = oracle.attention_gqa(q, k, v, 0.3, causal=causal)
    O_t, L_t = _sdpa(q, k, v, 0.3, causal)
    assert np.allclose(O, O_t, atol=1e-12) and np.allclose(L, L_t, atol=1e-12)


def test_group_of_one_is_multi_head():
    q, k, v = _rand(1, 5, 5, 40, 8, seed=1)
    O, L = oracle.attention_gqa(q, k, v, 0.5, causal=True)
    O2, L2 = oracle.attention(q, k, v, 0.5, causal=True)
    assert np.array_equal(O, O2) and np.array_equal(L, L2)


def test_each_query_head_against_its_kv_head():
    q, k, v = _rand(1, 6, 2, 9, 3, seed=2)
    O, L = oracle.attention_gqa(q, k, v, 0.7)
    for h in range(6):
        kv = h // 3
        Ob, Lb = oracle.attention_bruteforce(q[:, h:h + 1], k[:, kv:kv + 1], v[:, kv:kv + 1], 0.7)
        assert np.allclose(O[:, h:h + 1], Ob, atol=1e-13) and np.allclose(L[:, h:h + 1], Lb, atol=1e-13)


def test_same_query_in_one_group_gives_same_output():
    q, k, v = _rand(1, 4, 2, 20, 8, seed=3)
    q[:, 1] = q[:, 0]            # heads 0 and 1 share a group -> identical results
    q[:, 2] = q[:, 0]            # head 2 is in the other group -> different K/V
    O, L = oracle.attention_gqa(q, k, v, 0.4)
    assert np.array_equal(O[:, 0], O[:, 1]) and np.array_equal(L[:, 0], L[:, 1])
    assert not np.allclose(O[:, 0], O[:, 2])


def test_rejects_indivisible_heads():
    q, k, v = _rand(1, 6, 4, 8, 4, seed=4)
    with pytest.raises(ValueError):
        oracle.attention_gqa(q, k, v, 1.0)


@pytest.mark.parametrize("kind", ["interleaved", "reversed", "first_head_only"])
def test_pins_reject_wrong_head_mapping(kind):
    q, k, v = _rand(1, 8, 2, 30, 8, seed=5)

    def mutant(q, k, v, scale, causal=False):
        Hq, Hkv = q.shape[1], k.shape[1]
        if kind == "interleaved":
            kv = np.arange(Hq) % Hkv
        elif kind == "reversed":
            kv = (Hkv - 1) - np.arange(Hq) // (Hq // Hkv)
        else:
            kv = np.zeros(Hq, dtype=int)
        return oracle.attention(q.numpy(), k.numpy()[:, kv], v.numpy()[:, kv], scale, causal=causal)

    O_t, L_t = _sdpa(q, k, v, 0.3, False)
    O, L = mutant(q, k, v, 0.3)
    assert not (np.allclose(O, O_t, atol=1e-10) and np.allclose(L, L_t, atol=1e-10))
    O, L = oracle.attention_gqa(q, k, v, 0.3)
    assert np.allclose(O, O_t, atol=1e-12) and np.allclose(L, L_t, atol=1e-12)
