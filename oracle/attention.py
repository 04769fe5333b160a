"""CPU oracle for the FlashAttention-2 forward -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this module. The product path (the HIP library and its Python binding)
never imports, calls or links anything under oracle/.

Everything here is plain, slow float64 numpy written from the pages:

* attention() is the textbook definition FlashAttention reaches up to rounding
  order: the full score matrix S = scale * Q K^T is materialised row by row, the
  softmax is taken with the row max subtracted, and L is the natural-log
  logsumexp of the scaled scores.
  Sources: "Kernels and Memory in LLM Inference", section "Attention, said
  plainly again" (S = QK^T, row softmax, times V; subtract the row max);
  "FlashAttention-2 from PyTorch to Triton", the forward-pass section (L is the
  per-row logsumexp of the scaled scores) and its test file's reference
  function (SDPA output plus logsumexp of the scaled fp32 scores, causal mask
  keeps key <= query).

* attention_online() is a second, independent formulation: the FA-2 online
  softmax over key tiles (running max m, running sum l, rescale by
  exp(m_old - m_new), one divide at the end), in the order the PyTorch tiled
  implementation on "FlashAttention-2 from PyTorch to Triton" takes its steps.
  It exists to pin attention() by brute force on tiny inputs and to reproduce
  the worked example of "1.8x Faster Attention on an RTX 5080", section
  "The attention itself".

Readings where the pages are silent (each also listed in the design notes):
  - keys at index >= N do not exist (they are excluded, never zero-padded);
  - causal keeps key <= query, top-left aligned, square only;
  - L is the natural log; a row with no valid key would give O = 0 and
    L = -inf (it cannot occur for N >= 1 with this causal convention).
"""
from __future__ import annotations

import numpy as np


def _as_f64(x) -> np.ndarray:
    """Exact float64 copy of a numpy array or a CPU torch tensor (bf16 and fp32
    values are exactly representable in float64)."""
    try:
        import torch

        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover - torch is always present here
        pass
    return np.asarray(x, dtype=np.float64)


def attention(q, k, v, scale: float, causal: bool = False, rows=None):
    """O and L of softmax(scale * Q K^T) V for every (batch, head).

    q, k, v: [B, H, N, d] (any real dtype; upcast exactly to float64).
    rows: None for every query row, or an int array of query rows checked for
          every (batch, head).
    Returns (O [B, H, R, d] float64, L [B, H, R] float64) with R = number of
    rows.
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    B, H, N, d = q.shape
    assert k.shape == (B, H, N, d) and v.shape == (B, H, N, d)
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    R = rows.shape[0]
    O = np.zeros((B, H, R, d), dtype=np.float64)
    L = np.full((B, H, R), -np.inf, dtype=np.float64)
    key_idx = np.arange(N)
    for b in range(B):
        for h in range(H):
            # the selected rows of the score matrix, all N keys
            S = scale * (q[b, h, rows, :] @ k[b, h].T)
            if causal:
                S = np.where(key_idx[None, :] <= rows[:, None], S, -np.inf)
            m = S.max(axis=1, keepdims=True)
            valid = np.isfinite(m[:, 0])
            m_safe = np.where(np.isfinite(m), m, 0.0)
            E = np.exp(S - m_safe)                      # exp(-inf) = 0 for masked keys
            l = E.sum(axis=1, keepdims=True)
            Lrow = m_safe[:, 0] + np.log(np.where(valid, l[:, 0], 1.0))
            L[b, h] = np.where(valid, Lrow, -np.inf)
            P = np.where(valid[:, None], np.exp(S - np.where(valid, Lrow, 0.0)[:, None]), 0.0)
            O[b, h] = P @ v[b, h]
    return O, L


def attention_online(q, k, v, scale: float, causal: bool = False,
                     tile_q: int = 16, tile_k: int = 16, trace: bool = False):
    """The FA-2 forward as an online softmax over key tiles, in float64.

    For each query tile and each key tile in ascending order:
      S_ij  = scale * Q_i K_j^T, with keys >= N (and key > query if causal)
              set to -inf;
      m_new = max(m, rowmax S_ij);  P = exp(S_ij - m_new);
      alpha = exp(m - m_new);       l = alpha*l + rowsum P;
      O     = alpha*O + P V_j;      m = m_new;
    and finally O / l and L = m + log(l).

    With trace=True also returns, per (b, h, query row), the list of
    (m, l, alpha) after every key tile -- the quantities the worked example on
    "1.8x Faster Attention on an RTX 5080" prints.
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    B, H, N, d = q.shape
    O = np.zeros((B, H, N, d))
    L = np.zeros((B, H, N))
    traces = {}
    for b in range(B):
        for h in range(H):
            for q0 in range(0, N, tile_q):
                qi = np.arange(q0, min(q0 + tile_q, N))
                Qi = q[b, h, qi]
                m = np.full(len(qi), -np.inf)
                l = np.zeros(len(qi))
                Oi = np.zeros((len(qi), d))
                for k0 in range(0, N, tile_k):
                    kj = np.arange(k0, min(k0 + tile_k, N))
                    S = scale * (Qi @ k[b, h, kj].T)
                    if causal:
                        S = np.where(kj[None, :] <= qi[:, None], S, -np.inf)
                    m_new = np.maximum(m, S.max(axis=1))
                    # a row whose keys so far are all masked keeps m = -inf;
                    # exp(-inf - (-inf)) would be NaN, so such rows contribute 0
                    m_use = np.where(np.isfinite(m_new), m_new, 0.0)
                    P = np.exp(S - m_use[:, None])
                    alpha = np.where(np.isfinite(m_new), np.exp(m - m_use), 1.0)
                    l = alpha * l + P.sum(axis=1)
                    Oi = alpha[:, None] * Oi + P @ v[b, h, kj]
                    m = m_new
                    if trace:
                        for r, qrow in enumerate(qi):
                            traces.setdefault((b, h, int(qrow)), []).append(
                                (float(m[r]), float(l[r]), float(alpha[r])))
                O[b, h, qi] = Oi / l[:, None]
                L[b, h, qi] = m + np.log(l)
    if trace:
        return O, L, traces
    return O, L


def attention_bruteforce(q, k, v, scale: float, causal: bool = False):
    """Pure-Python loops with math.exp, for inputs of a few elements only."""
    import math

    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    B, H, N, d = q.shape
    O = np.zeros((B, H, N, d))
    L = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            for i in range(N):
                s = []
                for j in range(N):
                    if causal and j > i:
                        continue
                    dot = 0.0
                    for t in range(d):
                        dot += q[b, h, i, t] * k[b, h, j, t]
                    s.append((j, scale * dot))
                mx = max(x for _, x in s)
                z = sum(math.exp(x - mx) for _, x in s)
                L[b, h, i] = mx + math.log(z)
                for t in range(d):
                    O[b, h, i, t] = sum(math.exp(x - mx) / z * v[b, h, j, t] for j, x in s)
    return O, L
