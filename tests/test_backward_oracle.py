"""Pins for the attention backward oracle (CPU only).

attention_backward() is tied to things other than itself: torch's fp64
autograd through its own scaled-dot-product attention (an independent
library routine), central finite differences of <dO, O> built on the
pure-Python forward, closed forms (zero upstream gradient, a single key,
scale 0) and invariants of softmax (the dK rows of a head sum to zero, the dV
rows sum to the dO rows, D = rowsum(P * dP)). Planted mistakes in a copy of
the oracle must each fail a pin.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def _rand(B, H, N, d, seed):
    g = torch.Generator().manual_seed(seed)
    return [torch.randn((B, H, N, d), generator=g, dtype=torch.float64) for _ in range(4)]


def _autograd(q, k, v, do, scale, causal):
    q, k, v = (t.clone().requires_grad_(True) for t in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal, scale=scale)
    o.backward(do)
    return q.grad.numpy(), k.grad.numpy(), v.grad.numpy(), o.detach().numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 2, 37, 16), (2, 1, 64, 32), (1, 1, 1, 8)])
def test_matches_torch_autograd_fp64(causal, shape):
    q, k, v, do = _rand(*shape, seed=sum(shape))
    dq, dk, dv, D = oracle.attention_backward(q, k, v, do, 0.3, causal=causal)
    tq, tk, tv, to = _autograd(q, k, v, do, 0.3, causal)
    assert np.allclose(dq, tq, atol=1e-12) and np.allclose(dk, tk, atol=1e-12)
    assert np.allclose(dv, tv, atol=1e-12)
    assert np.allclose(D, np.sum(do.numpy() * to, axis=-1), atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_central_differences_of_the_pure_python_forward(causal):
    q, k, v, do = _rand(1, 1, 5, 3, seed=7)
    dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, 0.8, causal=causal)
    eps = 1e-6

    def loss(q_, k_, v_):
        O, _ = oracle.attention_bruteforce(q_, k_, v_, 0.8, causal=causal)
        return float(np.sum(O * do.numpy()))

    base = [t.numpy().copy() for t in (q, k, v)]
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        for idx in [(0, 0, 0, 0), (0, 0, 2, 1), (0, 0, 4, 2), (0, 0, 3, 0)]:
            plus = [t.copy() for t in base]
            minus = [t.copy() for t in base]
            plus[which][idx] += eps
            minus[which][idx] -= eps
            fd = (loss(*plus) - loss(*minus)) / (2 * eps)
            assert abs(fd - grad[idx]) < 1e-7, (which, idx, fd, grad[idx])


def test_softmax_invariants():
    q, k, v, do = _rand(2, 3, 50, 8, seed=3)
    for causal in (False, True):
        dq, dk, dv, D = oracle.attention_backward(q, k, v, do, 0.4, causal=causal)
        # shifting every key by one vector leaves softmax unchanged -> dK rows sum to 0
        assert np.allclose(dk.sum(axis=2), 0.0, atol=1e-12)
        # rows of P sum to 1 -> the dV rows sum to the dO rows
        assert np.allclose(dv.sum(axis=2), do.numpy().sum(axis=2), atol=1e-12)
        # D = rowsum(P * dP) = dO . O
        O, _ = oracle.attention(q, k, v, 0.4, causal=causal)
        assert np.allclose(D, np.sum(do.numpy() * O, axis=-1), atol=1e-12)


def test_closed_forms():
    q, k, v, do = _rand(1, 2, 20, 4, seed=4)
    # zero upstream gradient -> zero gradients
    dq, dk, dv, D = oracle.attention_backward(q, k, v, torch.zeros_like(do), 0.5)
    assert not np.any(dq) and not np.any(dk) and not np.any(dv) and not np.any(D)
    # one key: P = 1, O = v, dV = dO, and dS = dP - D = 0
    q1, k1, v1, do1 = _rand(1, 1, 1, 6, seed=5)
    dq, dk, dv, D = oracle.attention_backward(q1, k1, v1, do1, 0.9)
    assert np.allclose(dv, do1.numpy(), atol=1e-15)
    assert np.allclose(dq, 0, atol=1e-15) and np.allclose(dk, 0, atol=1e-15)
    # causal row 0 sees only key 0: its dQ row is zero
    dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, 0.5, causal=True)
    assert np.allclose(dq[:, :, 0], 0, atol=1e-15)
    # scale 0: dQ and dK carry the factor scale
    dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, 0.0)
    assert not np.any(dq) and not np.any(dk)
    assert np.allclose(dv, np.broadcast_to(do.numpy().mean(axis=2, keepdims=True), dv.shape), atol=1e-14)


def test_given_o_only_changes_d():
    q, k, v, do = _rand(1, 1, 30, 8, seed=6)
    O, _ = oracle.attention(q, k, v, 0.5)
    a = oracle.attention_backward(q, k, v, do, 0.5, o=O)
    b = oracle.attention_backward(q, k, v, do, 0.5)
    for x, y in zip(a, b):
        assert np.allclose(x, y, atol=1e-13)
    # a perturbed O moves D by exactly dO . delta
    delta = np.full_like(O, 1e-3)
    c = oracle.attention_backward(q, k, v, do, 0.5, o=O + delta)
    assert np.allclose(c[3] - b[3], np.sum(do.numpy() * delta, axis=-1), atol=1e-13)
    assert np.array_equal(c[2], b[2])       # dV does not use D


# --------------------------------------------------------------------------
# planted mistakes
# --------------------------------------------------------------------------
def _mutant(kind):
    def f(q, k, v, do, scale, causal=False, o=None):
        q, k, v, do = (t.numpy() if isinstance(t, torch.Tensor) else t for t in (q, k, v, do))
        B, H, N, d = q.shape
        out = [np.zeros_like(q), np.zeros_like(k), np.zeros_like(v), np.zeros((B, H, N))]
        for b in range(B):
            for h in range(H):
                S = scale * q[b, h] @ k[b, h].T
                if causal and kind != "causal_ignored":
                    S = np.where(np.tril(np.ones((N, N), bool)), S, -np.inf)
                E = np.exp(S - S.max(1, keepdims=True))
                P = E / E.sum(1, keepdims=True) if kind != "unnormalised" else E
                dP = do[b, h] @ v[b, h].T
                Dr = np.sum(P * dP, axis=1)
                dS = P * (dP - Dr[:, None]) if kind != "no_d" else P * dP
                out[0][b, h] = (scale if kind != "dq_no_scale" else 1.0) * dS @ k[b, h]
                out[1][b, h] = scale * (dS @ q[b, h] if kind == "ds_not_transposed" else dS.T @ q[b, h])
                out[2][b, h] = P.T @ do[b, h]
                out[3][b, h] = Dr
        return tuple(out)
    return f


def _pins_pass(fn) -> bool:
    try:
        for causal in (False, True):
            q, k, v, do = _rand(1, 2, 24, 24, seed=11)
            got = fn(q, k, v, do, 0.3, causal=causal)
            ref = _autograd(q, k, v, do, 0.3, causal)
            if not all(np.allclose(g, r, atol=1e-10) for g, r in zip(got[:3], ref[:3])):
                return False
        return True
    except Exception:
        return False


def test_pins_accept_the_oracle():
    assert _pins_pass(oracle.attention_backward)


@pytest.mark.parametrize("kind", ["no_d", "ds_not_transposed", "dq_no_scale", "unnormalised",
                                  "causal_ignored"])
def test_pins_reject_planted_mistake(kind):
    assert not _pins_pass(_mutant(kind))


@pytest.mark.parametrize("causal", [False, True])
def test_sampled_rows_agree_with_the_full_backward(causal):
    q, k, v, do = _rand(2, 3, 70, 8, seed=12)
    O, _ = oracle.attention(q, k, v, 0.35, causal=causal)
    dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, 0.35, causal=causal, o=O)
    q_rows = np.array([0, 1, 33, 69])
    k_rows = np.array([0, 5, 40, 69])
    heads = [(0, 0), (1, 2)]
    sq, sk, sv = oracle.attention_backward_rows(q, k, v, do, 0.35, causal, O, q_rows, k_rows,
                                                heads=heads, chunk=16)
    for t, (b, h) in enumerate(heads):
        assert np.allclose(sq[t], dq[b, h, q_rows], atol=1e-12)
        assert np.allclose(sk[t], dk[b, h, k_rows], atol=1e-12)
        assert np.allclose(sv[t], dv[b, h, k_rows], atol=1e-12)
