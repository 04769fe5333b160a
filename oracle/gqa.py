"""Grouped-query attention -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this module; the product path never imports, calls or links it. Plain
float64 numpy.

Source: "Kernels and Memory in LLM Inference", section "Store less: MQA, GQA,
MLA". The query heads are split into groups and every group shares one key
head and one value head; one group is multi-query attention, one group per
query head is ordinary multi-head attention. Reading taken where the page is
silent: the groups are runs of consecutive query heads, so with Hq query heads
and Hkv key/value heads, query head h uses key/value head h // (Hq / Hkv).

attention_gqa() is that definition written out: every query head runs the
plain attention() of this package against its group's K and V.
"""
from __future__ import annotations

import numpy as np

from .attention import _as_f64, attention


def kv_head_of(Hq: int, Hkv: int) -> np.ndarray:
    """Key/value head used by each of the Hq query heads."""
    if Hkv < 1 or Hq % Hkv != 0:
        raise ValueError("the number of query heads must be a multiple of the key/value heads")
    return np.arange(Hq) // (Hq // Hkv)


def attention_gqa(q, k, v, scale: float, causal: bool = False, rows=None):
    """O [B, Hq, R, d] and L [B, Hq, R] for q [B, Hq, N, d] and k, v
    [B, Hkv, N, d]."""
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    kv = kv_head_of(q.shape[1], k.shape[1])
    return attention(q, k[:, kv], v[:, kv], scale, causal=causal, rows=rows)
