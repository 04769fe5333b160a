"""CPU oracle for the per-head FP8-e4m3 quantiser -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this module.

"1.8x Faster Attention on an RTX 5080" (section "Who am I, what's mine?")
quantises Q, K and V per head to FP8 and carries one fp32 descale per head and
tensor, folding them into the two scalars qk_scale = dq * dk * softmax_scale and
pv_scale = dv / 256. The page does not spell out the format or the arithmetic.
The readings taken here:
  - the format is OCP e4m3fn: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa
    bits, largest finite value 448, codes 0x7F / 0xFF are NaN, no infinity;
  - per (batch, head): amax = max |x| in fp32, descale = fp32(amax / 448),
    mult = fp32(448 / amax) (each a correctly rounded fp32 division),
    code = e4m3_rne(clamp(fp32(x * mult), -448, 448));
  - amax == 0 gives descale = mult = 1.

The e4m3 rounding is written from the format's definition: the table of every
finite e4m3fn value is enumerated from its bit fields, and a value is rounded
to the nearest entry, ties going to the entry whose code is even (the one with
a zero last mantissa bit).
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_table() -> np.ndarray:
    """float64 value of every code 0..255 (NaN for 0x7F and 0xFF)."""
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            vals[code] = np.nan
        elif e == 0:
            vals[code] = sign * (m / 8.0) * 2.0 ** (1 - 7)      # subnormal
        else:
            vals[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_TABLE = e4m3_table()
# non-negative finite codes 0x00..0x7E in increasing value order
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALS = _TABLE[:0x7F]
assert np.all(np.diff(_POS_VALS) > 0)


def e4m3_encode(x) -> np.ndarray:
    """Round finite values with |x| <= 448 to the nearest e4m3fn code (ties to
    the even code). Returns uint8 codes of x's shape."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(~np.isfinite(x)) or np.any(np.abs(x) > E4M3_MAX):
        raise ValueError("e4m3_encode expects finite values within [-448, 448]")
    a = np.abs(x).ravel()
    hi = np.searchsorted(_POS_VALS, a, side="left")       # first entry >= a
    hi = np.clip(hi, 0, len(_POS_VALS) - 1)
    lo = np.clip(hi - 1, 0, None)
    d_lo = a - _POS_VALS[lo]
    d_hi = _POS_VALS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))
    exact = _POS_VALS[hi] == a
    code = np.where(exact | pick_hi, _POS_CODES[hi], _POS_CODES[lo])
    # the sign bit is kept, also when the magnitude rounds to zero (-0)
    code = np.where(np.signbit(x.ravel()), code | 0x80, code)
    return code.astype(np.uint8).reshape(x.shape)


def e4m3_decode(codes) -> np.ndarray:
    return _TABLE[np.asarray(codes, dtype=np.uint8).astype(np.int64)]


def quantize_per_head(x):
    """x: [B, H, N, d] (bf16 / fp32 values; a torch tensor or numpy array).
    Returns (codes uint8 [B, H, N, d], descale float32 [B, H])."""
    try:
        import torch

        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu", torch.float32).numpy()
    except ImportError:  # pragma: no cover
        pass
    x = np.asarray(x, dtype=np.float32)
    B, H, N, d = x.shape
    codes = np.empty(x.shape, dtype=np.uint8)
    descale = np.empty((B, H), dtype=np.float32)
    for b in range(B):
        for h in range(H):
            xs = x[b, h]
            amax = np.float32(np.max(np.abs(xs))) if xs.size else np.float32(0.0)
            if amax == 0:
                ds, mult = np.float32(1.0), np.float32(1.0)
            else:
                # float64 quotient of two fp32 values rounded once to fp32 is the
                # correctly rounded fp32 quotient (53 >= 2*24 + 2)
                ds = np.float32(np.float64(amax) / E4M3_MAX)
                mult = np.float32(E4M3_MAX / np.float64(amax))
            # the product of two fp32 values is exact in float64; one rounding
            # to fp32 gives the fp32 product
            y = (xs.astype(np.float64) * np.float64(mult)).astype(np.float32)
            y = np.clip(y.astype(np.float64), -E4M3_MAX, E4M3_MAX)
            codes[b, h] = e4m3_encode(y)
            descale[b, h] = ds
    return codes, descale


def dequantize_per_head(codes, descale) -> np.ndarray:
    """float64 values code_value * descale, per (batch, head)."""
    vals = e4m3_decode(codes)
    return vals * np.asarray(descale, dtype=np.float64)[:, :, None, None]
