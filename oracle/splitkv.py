"""Split-KV partials and their merge -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this module; the product path never imports, calls or links it. Plain,
slow float64 numpy.

Source: "Kernels and Memory in LLM Inference", section "Flash-Decoding: one
token, whole chip". The keys are cut into contiguous chunks; each chunk's
attention is formed on its own, with its own running max and running sum; a
second step merges the partial results, rescaling each by how far its own max
lies below the overall max, and the merged result is exact attention.

* attention_keyrange() is the plain definition (attention() in this package)
  restricted to the keys k0 <= j < k1: it returns the chunk's output already
  divided by the chunk's own sum, O_s, and the chunk's natural-log logsumexp,
  L_s = m_s + log l_s. A query row with no valid key in the chunk (the chunk
  is empty, or lies wholly above the row under the causal mask) gets O_s = 0
  and L_s = -inf.

* merge_partials() is the merge step written in that (O_s, L_s) form. A chunk
  with max m_s, sum l_s and unnormalised output A_s has O_s = A_s / l_s and
  exp(m_s - M) l_s = exp(L_s - M); so rescaling the chunks to a common max M
  gives O = sum_s exp(L_s - M) O_s / sum_s exp(L_s - M) and
  L = M + log sum_s exp(L_s - M). Any common M gives the same result; the
  largest L_s is used so that no weight exceeds 1. Chunks with L_s = -inf
  weigh nothing; a row with every L_s = -inf stays O = 0, L = -inf.
"""
from __future__ import annotations

import numpy as np

from .attention import _as_f64


def attention_keyrange(q, k, v, scale: float, causal: bool, k0: int, k1: int, rows=None):
    """O_s [B, H, R, d] and L_s [B, H, R] of softmax(scale * Q K^T) V over the
    keys k0 <= j < min(k1, N) only (causal keeps j <= query row as well)."""
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    B, H, N, d = q.shape
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    R = rows.shape[0]
    O = np.zeros((B, H, R, d), dtype=np.float64)
    L = np.full((B, H, R), -np.inf, dtype=np.float64)
    keys = np.arange(max(k0, 0), min(k1, N))
    if keys.size == 0:
        return O, L
    for b in range(B):
        for h in range(H):
            S = scale * (q[b, h, rows, :] @ k[b, h, keys, :].T)
            if causal:
                S = np.where(keys[None, :] <= rows[:, None], S, -np.inf)
            m = S.max(axis=1)
            valid = np.isfinite(m)
            m_safe = np.where(valid, m, 0.0)
            E = np.exp(S - m_safe[:, None])
            l = E.sum(axis=1)
            Lrow = np.where(valid, m_safe + np.log(np.where(valid, l, 1.0)), -np.inf)
            P = np.where(valid[:, None], E / np.where(valid, l, 1.0)[:, None], 0.0)
            O[b, h] = P @ v[b, h, keys, :]
            L[b, h] = Lrow
    return O, L


def merge_partials(O_parts, L_parts):
    """Merge S partials: O_parts [S, ..., d], L_parts [S, ...] -> (O, L)."""
    O_parts = np.asarray(O_parts, dtype=np.float64)
    L_parts = np.asarray(L_parts, dtype=np.float64)
    M = L_parts.max(axis=0)
    valid = np.isfinite(M)
    M_safe = np.where(valid, M, 0.0)
    w = np.exp(L_parts - M_safe[None])              # exp(-inf) = 0 for empty chunks
    z = w.sum(axis=0)
    z_safe = np.where(valid, z, 1.0)
    O = (w[..., None] * O_parts).sum(axis=0) / z_safe[..., None]
    O = np.where(valid[..., None], O, 0.0)
    L = np.where(valid, M_safe + np.log(z_safe), -np.inf)
    return O, L
