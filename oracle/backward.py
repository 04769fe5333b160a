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
