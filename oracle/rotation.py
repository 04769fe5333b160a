"""Rotation of Q and K before FP8 quantisation -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this module; the product path never imports, calls or links it.

Source: "Kernels and Memory in LLM Inference", section "Precision: FP8 with a
real failure mode": FP8 quantisation of transformer activations fails on a
few large outlier coordinates; FlashAttention-3's second answer multiplies Q
and K by a fixed random rotation before quantising, which spreads the loud
coordinates over all dimensions and leaves Q K^T unchanged (the rotations
cancel). Readings taken where the page is silent:
  - the rotation is a randomised Hadamard transform: x -> (x * s) H, with s a
    vector of d random signs (an input; the same s for Q and K) and H the
    d x d Sylvester Hadamard matrix, H_ij = (-1)^popcount(i & j), left
    unnormalised (H H^T = d I), so rotated Q times rotated K^T is d Q K^T;
  - the rotated values are rounded once to fp32 from their exact sums (bf16
    inputs: every partial sum of at most d = 128 signed bf16 values is exact
    in float64 unless a row spans more than 38 binary orders of magnitude),
    then quantised per head exactly as quantize_per_head() does;
  - the factor d is taken out of Q's descale (an exact power of two), so the
    FP8 attention on the rotated codes needs no other change.
"""
from __future__ import annotations

import numpy as np

from .fp8 import quantize_per_head


def hadamard(d: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order d (a power of two): H_1 = [1],
    H_2n = [[H, H], [H, -H]]."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    H = np.ones((1, 1))
    while H.shape[0] < d:
        H = np.block([[H, H], [H, -H]])
    return H


def rotate(x, signs) -> np.ndarray:
    """(x * signs) H along the last axis, exact in float64 for bf16 inputs,
    rounded once to float32. x: [..., d]; signs: d values of +1 / -1."""
    try:
        import torch

        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    x = np.asarray(x, dtype=np.float64)
    s = np.asarray(signs, dtype=np.float64)
    d = x.shape[-1]
    assert s.shape == (d,) and np.all(np.abs(s) == 1)
    return ((x * s) @ hadamard(d)).astype(np.float32)


def quantize_rotated(x, signs, fold_inverse_d: bool):
    """Rotate, then quantise per head. Returns (codes uint8 [B, H, N, d],
    descale float32 [B, H]); with fold_inverse_d the descale carries the 1/d
    that undoes H H^T = d I (used for Q)."""
    y = rotate(x, signs)
    codes, descale = quantize_per_head(y)
    if fold_inverse_d:
        descale = (descale / np.float32(y.shape[-1])).astype(np.float32)
    return codes, descale
