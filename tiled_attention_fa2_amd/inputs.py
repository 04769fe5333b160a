"""Seeded synthetic inputs for the attention forward.

This module only draws random numbers and shapes them. It holds none of the
attention or quantisation arithmetic, so the CPU oracle and the HIP path can
both be fed from it without sharing any of the method.

Workloads follow the shapes the pages measure on: the MiniMax H3 DiT block's
self-attention (56 heads x 30272 tokens x head dim 128) from "1.8x Faster
Attention on an RTX 5080", section "The attention itself", plus the small and
causal shapes used for parity. The real activations are not available; iid
N(0, 1) tensors of the same shapes stand in for them.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str          # "f32", "bf16" or "fp8" (fp8 = bf16 draws quantised per head)
    B: int
    H: int
    N: int
    d: int
    causal: bool
    Hkv: int = 0        # key/value heads (grouped-query attention); 0 = H

    @property
    def kv_heads(self) -> int:
        return self.Hkv or self.H

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def flops(self) -> float:
        """4*B*H*N^2*d, halved for causal (the pages' accounting)."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2 if self.causal else f


WORKLOADS = {
    w.name: w
    for w in (
        Workload("f32_b1_h1_n256_d64", "f32", 1, 1, 256, 64, False),
        Workload("bf16_b1_h8_n4096_d128", "bf16", 1, 8, 4096, 128, False),
        Workload("bf16_causal_b4_h32_n2048_d128", "bf16", 4, 32, 2048, 128, True),
        Workload("bf16_dit_b1_h56_n30272_d128", "bf16", 1, 56, 30272, 128, False),
        Workload("fp8_dit_b1_h56_n30272_d128", "fp8", 1, 56, 30272, 128, False),
        # the DiT shape with grouped-query attention: 56 query heads over 8
        # key/value heads ("Kernels and Memory in LLM Inference", section
        # "Store less: MQA, GQA, MLA"; about 8 groups is the setting it names)
        Workload("bf16_gqa_b1_hq56_hkv8_n30272_d128", "bf16", 1, 56, 30272, 128, False, Hkv=8),
        # one GPU's share of the DiT shape when its 56 heads are split over 8
        # GPUs: 7 heads
        Workload("bf16_dit_shard_b1_h7_n30272_d128", "bf16", 1, 7, 30272, 128, False),
        Workload("fp8_dit_shard_b1_h7_n30272_d128", "fp8", 1, 7, 30272, 128, False),
        # the DiT shape at head dim 64 (the other head dim the library takes)
        Workload("bf16_dit_b1_h56_n30272_d64", "bf16", 1, 56, 30272, 64, False),
        Workload("fp8_dit_b1_h56_n30272_d64", "fp8", 1, 56, 30272, 64, False),
    )
}


def make_qkv(B: int, H: int, N: int, d: int, dtype: str = "bf16", seed: int = 0,
             variant: str = "iid"):
    """Draw Q, then K, then V as iid N(0,1) float32 on the CPU with one seeded
    generator, then round to bf16 unless dtype == "f32".

    variant shapes the draws for stress cases (all still seeded):
      "iid"      plain N(0,1)
      "peaked"   Q multiplied by 8: near one-hot rows, frequent rescales
      "growing"  key norms rise along the sequence, so the running max rises
                 on almost every key tile
      "outlier"  a few channels of Q, K and V multiplied by 20 (the kind of
                 outliers that make fp8 hard)
    """
    g = torch.Generator().manual_seed(seed)
    shape = (B, H, N, d)
    q = torch.randn(shape, generator=g, dtype=torch.float32)
    k = torch.randn(shape, generator=g, dtype=torch.float32)
    v = torch.randn(shape, generator=g, dtype=torch.float32)
    if variant == "peaked":
        q = q * 8.0
    elif variant == "growing":
        ramp = torch.linspace(0.25, 3.0, N, dtype=torch.float32).view(1, 1, N, 1)
        k = k * ramp
    elif variant == "outlier":
        ch = torch.randperm(d, generator=g)[: max(1, d // 32)]
        for t in (q, k, v):
            t[..., ch] *= 20.0
    elif variant != "iid":
        raise ValueError(f"unknown variant {variant!r}")
    if dtype == "f32":
        return q, k, v
    if dtype in ("bf16", "fp8"):
        return q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)
    raise ValueError(f"unknown dtype {dtype!r}")


def make_qkv_long(N: int, d: int, seed: int = 0, chunk_rows: int = 1 << 18, threads: int = 16):
    """One head (B = H = 1) of bf16 Q, K, V for sequences too long for one
    sequential generator: rows [c*chunk_rows, (c+1)*chunk_rows) of tensor t
    (0 = Q, 1 = K, 2 = V) are iid N(0,1) float32 from a generator seeded with
    (seed * 3 + t) * 2^20 + c, rounded to bf16. Chunks are drawn on a thread
    pool; the result depends only on (N, d, seed, chunk_rows)."""
    from concurrent.futures import ThreadPoolExecutor

    assert N >= 0 and chunk_rows > 0
    out = [torch.empty((1, 1, N, d), dtype=torch.bfloat16) for _ in range(3)]
    n_chunks = (N + chunk_rows - 1) // chunk_rows

    def draw(job):
        t, c = job
        g = torch.Generator().manual_seed((seed * 3 + t) * (1 << 20) + c)
        r0, r1 = c * chunk_rows, min(N, (c + 1) * chunk_rows)
        out[t][0, 0, r0:r1] = torch.randn((r1 - r0, d), generator=g, dtype=torch.float32).to(torch.bfloat16)

    with ThreadPoolExecutor(max_workers=threads) as pool:
        list(pool.map(draw, [(t, c) for t in range(3) for c in range(n_chunks)]))
    return tuple(out)


def make_gqa(B: int, Hq: int, Hkv: int, N: int, d: int, dtype: str = "bf16", seed: int = 0):
    """Q with Hq heads, then K and V with Hkv heads: iid N(0,1) float32 from one
    seeded generator in that order, rounded to bf16 unless dtype == "f32"."""
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((B, Hq, N, d), generator=g, dtype=torch.float32)
    k = torch.randn((B, Hkv, N, d), generator=g, dtype=torch.float32)
    v = torch.randn((B, Hkv, N, d), generator=g, dtype=torch.float32)
    if dtype == "f32":
        return q, k, v
    if dtype in ("bf16", "fp8"):
        return q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)
    raise ValueError(f"unknown dtype {dtype!r}")


def make_workload(name: str, seed: int = 0, variant: str = "iid"):
    w = WORKLOADS[name]
    if w.kv_heads != w.H:
        return w, make_gqa(w.B, w.H, w.kv_heads, w.N, w.d, w.dtype, seed=seed)
    return w, make_qkv(w.B, w.H, w.N, w.d, w.dtype, seed=seed, variant=variant)


def sample_rows(N: int, tile: int = 128, n_random: int = 64, seed: int = 12345):
    """Query rows checked at full size: rows 0, 1, N-1, every row of the last
    (ragged) query tile and n_random uniform draws, sorted and unique."""
    import numpy as np

    rng = np.random.default_rng(seed)
    last_tile_start = ((N - 1) // tile) * tile
    rows = {0, 1, N - 1}
    rows.update(range(last_tile_start, N))
    rows.update(int(r) for r in rng.integers(0, N, size=n_random))
    return np.array(sorted(r for r in rows if 0 <= r < N), dtype=np.int64)


def make_partials(S: int, BH: int, N: int, d: int, seed: int = 0, p_empty: float = 0.3,
                  spread: float = 10.0):
    """Seeded stand-ins for S partial attention results over disjoint key sets:
    o_parts float32 [S, BH, N, d] ~ N(0, 4), lse_parts float32 [S, BH, N] ~
    N(0, spread^2). A fraction p_empty of the (part, row) entries is empty
    (L = -inf, O = 0); rows 0..4 of the first head are empty in every part; the
    second head's first part is shifted up by 500 (weights far apart)."""
    g = torch.Generator().manual_seed(seed)
    o = torch.randn((S, BH, N, d), generator=g, dtype=torch.float32) * 2.0
    lse = torch.randn((S, BH, N), generator=g, dtype=torch.float32) * spread
    empty = torch.rand((S, BH, N), generator=g) < p_empty
    empty[:, 0, :5] = True
    if BH > 1:
        lse[0, 1] += 500.0
    lse[empty] = float("-inf")
    o[empty] = 0.0
    return o, lse


def make_dout(B: int, H: int, N: int, d: int, seed: int = 0):
    """Upstream gradient dO for the backward: iid N(0,1) float32 from its own
    seeded generator, rounded to bf16."""
    g = torch.Generator().manual_seed(seed)
    return torch.randn((B, H, N, d), generator=g, dtype=torch.float32).to(torch.bfloat16)


def make_signs(d: int, seed: int = 0):
    """The d random signs of a randomised Hadamard rotation, drawn from their
    own seeded generator: int8 [d] of +1 / -1, each with probability 1/2."""
    g = torch.Generator().manual_seed(seed)
    bits = torch.randint(0, 2, (d,), generator=g, dtype=torch.int64)
    return (1 - 2 * bits).to(torch.int8)
