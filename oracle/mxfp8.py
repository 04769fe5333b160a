"""Per-block FP8 scales -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this module; the product path never imports, calls or links it. Plain
float64 numpy, with the e4m3 rounding of fp8.py.

Source: "Kernels and Memory in LLM Inference", section "Precision: FP8 with a
real failure mode": one scale for a whole tensor is stretched by its few
outliers until the many small values share a handful of FP8 levels; the first
remedy FlashAttention-3 uses is a separate scale for every block, so an
outlier only coarsens the grid of its own block.

Readings taken where the page is silent (block shape, scale format, rounding):
  - a block is 32 consecutive elements along the axis that the product it
    feeds sums over, as in the OCP microscaling (MX) formats: Q and K are cut
    into blocks of 32 elements of one row (S = Q K^T sums over the head
    dimension), V into blocks of 32 keys of one column (O = P V sums over the
    keys); a ragged last block of V holds the keys that remain;
  - every scale is a power of two 2^e, stored as the E8M0 byte e + 127;
  - e is the smallest integer with amax(block) <= 448 * 2^e, so no element
    saturates and the block's largest magnitude lands in (224, 448]; e is
    clamped to [-127, 127] (an all-zero block gets -127);
  - each element's code is e4m3 round-to-nearest-even of x * 2^-e, and its
    value is that code's value times 2^e.
"""
from __future__ import annotations

import numpy as np

from .fp8 import E4M3_MAX, e4m3_decode, e4m3_encode

ROW_BLOCK = 32      # Q, K: elements of one row per block
KEY_BLOCK = 32      # V: keys of one column per block
E_MIN, E_MAX = -127, 127


def _as_f64(x) -> np.ndarray:
    try:
        import torch

        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def mx_exponent(amax) -> np.ndarray:
    """Smallest integer e with amax <= 448 * 2^e, clamped to [-127, 127]
    (int64 array of amax's shape; amax >= 0, exact in float64)."""
    a = np.asarray(amax, dtype=np.float64)
    if np.any(a < 0) or np.any(~np.isfinite(a)):
        raise ValueError("amax must be finite and non-negative")
    _, e2 = np.frexp(a)                      # a = f 2^e2, f in [0.5, 1)
    e = e2.astype(np.int64) - 9              # a first guess, within one of the answer
    # step up while the bound fails, then down while the one below still holds
    for _ in range(3):
        e = np.where(a > np.ldexp(E4M3_MAX, e), e + 1, e)
    for _ in range(3):
        e = np.where(a <= np.ldexp(E4M3_MAX, e - 1), e - 1, e)
    e = np.where(a == 0.0, E_MIN, e)
    return np.clip(e, E_MIN, E_MAX)


def _quantize_blocks(blocks: np.ndarray):
    """blocks [..., n]: one block per last-axis vector. Returns (codes uint8
    [..., n], E8M0 bytes uint8 [...])."""
    e = mx_exponent(np.max(np.abs(blocks), axis=-1))
    scaled = np.ldexp(blocks, -e[..., None])          # exact: a power of two
    codes = e4m3_encode(scaled)
    return codes, (e + 127).astype(np.uint8)


def quantize_mx(x, axis: str):
    """Per-block e4m3 quantisation of x [B, H, N, d].

    axis "rows": blocks of 32 consecutive elements of a row (Q, K); returns
      (codes uint8 [B, H, N, d], scales uint8 [B, H, N, d / 32]).
    axis "keys": blocks of 32 consecutive keys of a column (V); returns
      (codes uint8 [B, H, N, d], scales uint8 [B, H, ceil(N / 32), d])."""
    x = _as_f64(x)
    B, H, N, d = x.shape
    if axis == "rows":
        if d % ROW_BLOCK:
            raise ValueError("d must be a multiple of 32")
        codes, scales = _quantize_blocks(x.reshape(B, H, N, d // ROW_BLOCK, ROW_BLOCK))
        return codes.reshape(B, H, N, d), scales
    if axis == "keys":
        nc = -(-N // KEY_BLOCK)
        codes = np.zeros((B, H, N, d), dtype=np.uint8)
        scales = np.zeros((B, H, nc, d), dtype=np.uint8)
        for c in range(nc):
            k0, k1 = c * KEY_BLOCK, min(N, (c + 1) * KEY_BLOCK)
            blk = np.moveaxis(x[:, :, k0:k1, :], 2, -1)          # [B, H, d, keys]
            cb, sb = _quantize_blocks(blk)
            codes[:, :, k0:k1, :] = np.moveaxis(cb, -1, 2)
            scales[:, :, c, :] = sb
        return codes, scales
    raise ValueError(f"unknown axis {axis!r}")


def dequantize_mx(codes, scales, axis: str) -> np.ndarray:
    """float64 values code * 2^(scale - 127) for quantize_mx's output."""
    vals = e4m3_decode(np.asarray(codes))
    e = np.asarray(scales).astype(np.int64) - 127
    B, H, N, d = vals.shape
    if axis == "rows":
        return np.ldexp(vals, np.repeat(e, ROW_BLOCK, axis=-1))
    if axis == "keys":
        return np.ldexp(vals, np.repeat(e, KEY_BLOCK, axis=2)[:, :, :N, :])
    raise ValueError(f"unknown axis {axis!r}")


def quantize_qkv_mx(q, k, v):
    """Q and K by rows, V by keys. Returns ((q8, qs), (k8, ks), (v8, vs))."""
    return quantize_mx(q, "rows"), quantize_mx(k, "rows"), quantize_mx(v, "keys")


def quantize_rotated_mx(x, signs, fold_inverse_d: bool):
    """Row blocks of the randomised Hadamard rotation of x (rotation.rotate:
    exact float64 sums rounded once to fp32), multiplied in fp32 by the power
    of two 1/d when fold_inverse_d (for Q: the rotations of Q and K then
    cancel exactly in Q K^T). Returns quantize_mx(..., "rows")'s output."""
    from .rotation import rotate

    y = rotate(x, signs)
    if fold_inverse_d:
        y = (y * np.float32(1.0 / y.shape[-1])).astype(np.float32)
    return quantize_mx(y, "rows")
