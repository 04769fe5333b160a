"""Backward pass of attention -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this module; the product path never imports, calls or links it. Plain,
slow float64 numpy.

Sources: "FlashAttention-2 from PyTorch to Triton", forward-pass section (the
stored L lets the backward recompute P = exp(S - L) tile by tile) and its list
of what the first kernel leaves out (the tiled backward needs L, the row
quantity D = rowsum(dO * O), a pass over query tiles for every key tile that
builds dK and dV, and dQ from atomics or a second pass); "Kernels and Memory in
LLM Inference", section "Training detour (brief)" (the backward reloads Q, K,
V and recomputes each attention tile instead of storing it).

attention_backward() is the gradient of the definition written out, the
result the tiled backward reaches up to rounding order. With S = scale Q K^T
(keys after the query masked when causal), P = softmax(S) row by row and
O = P V, for an upstream gradient dO:
    dV = P^T dO,
    dP = dO V^T,
    D_i = sum_j P_ij dP_ij = dO_i . O_i      (the row quantity above),
    dS = P * (dP - D)                         (softmax's Jacobian, row by row),
    dQ = scale dS K,   dK = scale dS^T Q.
Reading taken where the pages are silent: D is formed from the O the caller
passes (the stored forward output, as a tiled backward reads it); without one
the exact O is used. L is an auxiliary output and takes no gradient.
"""
from __future__ import annotations

import numpy as np

from .attention import _as_f64


def attention_backward(q, k, v, do, scale: float, causal: bool = False, o=None):
    """Returns (dQ, dK, dV, D): dQ, dK, dV [B, H, N, d] and D [B, H, N]."""
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    do = _as_f64(do)
    o_given = None if o is None else _as_f64(o)
    B, H, N, d = q.shape
    dQ = np.zeros_like(q)
    dK = np.zeros_like(k)
    dV = np.zeros_like(v)
    D = np.zeros((B, H, N))
    keep = np.tril(np.ones((N, N), dtype=bool)) if causal else np.ones((N, N), dtype=bool)
    for b in range(B):
        for h in range(H):
            S = scale * (q[b, h] @ k[b, h].T)
            S = np.where(keep, S, -np.inf)
            m = S.max(axis=1, keepdims=True)
            E = np.exp(S - m)
            P = E / E.sum(axis=1, keepdims=True)
            O = P @ v[b, h] if o_given is None else o_given[b, h]
            dV[b, h] = P.T @ do[b, h]
            dP = do[b, h] @ v[b, h].T
            Dr = np.sum(do[b, h] * O, axis=1)
            dS = P * (dP - Dr[:, None])
            dQ[b, h] = scale * (dS @ k[b, h])
            dK[b, h] = scale * (dS.T @ q[b, h])
            D[b, h] = Dr
    return dQ, dK, dV, D


def attention_backward_rows(q, k, v, do, scale: float, causal: bool, o, q_rows, k_rows,
                            heads=None, chunk: int = 1024):
    """The gradients of attention_backward() evaluated only where asked: dQ at
    the query rows q_rows and dK, dV at the key rows k_rows, for the (batch,
    head) pairs in `heads` (default: all), for shapes whose full score matrix
    does not fit in memory. q, k, v, do, o: [B, H, N, d] (K/V with as many
    heads as Q). Every query row's logsumexp L comes from attention() over
    `chunk` rows at a time; then P_ij = exp(S_ij - L_i), D_i = dO_i . O_i and
    the same formulas as attention_backward().
    Returns (dQ [P, Rq, d], dK [P, Rk, d], dV [P, Rk, d]) for the P pairs."""
    from .attention import attention

    B, H, N, d = q.shape
    q_rows = np.asarray(q_rows, dtype=np.int64)
    k_rows = np.asarray(k_rows, dtype=np.int64)
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    dQ = np.zeros((len(pairs), len(q_rows), d))
    dK = np.zeros((len(pairs), len(k_rows), d))
    dV = np.zeros((len(pairs), len(k_rows), d))
    keys = np.arange(N)
    for t, (b, h) in enumerate(pairs):
        # one (batch, head) at a time, upcast exactly to float64
        qh, kh, vh, doh, oh = (_as_f64(x[b:b + 1, h:h + 1])[0, 0] for x in (q, k, v, do, o))
        L = np.concatenate([attention(qh[None, None], kh[None, None], vh[None, None], scale,
                                      causal=causal, rows=np.arange(r0, min(N, r0 + chunk)))[1][0, 0]
                            for r0 in range(0, N, chunk)])
        D = np.sum(doh * oh, axis=1)
        # query rows: dQ_i = scale sum_j P_ij (dP_ij - D_i) k_j
        S = scale * (qh[q_rows] @ kh.T)
        if causal:
            S = np.where(keys[None, :] <= q_rows[:, None], S, -np.inf)
        P = np.exp(S - L[q_rows, None])
        dP = doh[q_rows] @ vh.T
        dQ[t] = scale * ((P * (dP - D[q_rows, None])) @ kh)
        # key rows: dV_j = sum_i P_ij dO_i, dK_j = scale sum_i P_ij (dP_ij - D_i) q_i
        St = scale * (kh[k_rows] @ qh.T)          # [Rk, N] = S^T at the key rows
        if causal:
            St = np.where(keys[None, :] >= k_rows[:, None], St, -np.inf)
        Pt = np.exp(St - L[None, :])
        dPt = vh[k_rows] @ doh.T
        dV[t] = Pt @ doh
        dK[t] = scale * ((Pt * (dPt - D[None, :])) @ qh)
    return dQ, dK, dV
