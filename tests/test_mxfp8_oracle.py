"""Pins for the per-block FP8 oracle (CPU only).

"Kernels and Memory in LLM Inference", section "Precision: FP8 with a real
failure mode": a scale per block keeps one outlier from coarsening every other
value's grid. quantize_mx() is tied to things other than itself: the exponent
against an exact search over all E8M0 exponents with rational arithmetic; the
codes and scales against a pure-Python loop over the blocks (which fixes the
block axis, size and the ragged last block); the error bound of e4m3 rounding
(half a spacing); exact round trips of representable values; the isolation of
blocks from each other's outliers; the failure mode itself (a near-zero
majority keeps its precision per block and loses it under one scale per
head). Planted mistakes in copies of the quantiser must each fail a pin.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle.mxfp8 import KEY_BLOCK, ROW_BLOCK

E4M3_VALUES = oracle.e4m3_table()


def _exponent_search(a: float) -> int:
    """Smallest e in [-127, 127] with a <= 448 2^e (exact rationals); -127 if
    every e works, 127 if none does."""
    fa = Fraction(a)
    for e in range(-127, 128):
        if fa <= 448 * Fraction(2) ** e:
            return e
    return 127


def test_exponent_matches_exact_search():
    vals = [0.0, 1.0, 448.0, 449.0, 224.0, 256.0, 3.0e38, 1e-30, 2.0 ** -149, 2.0 ** -126]
    for k in range(-140, 120, 7):
        b = 448.0 * 2.0 ** k
        vals += [b, np.nextafter(b, 0.0), np.nextafter(b, np.inf), 2.0 ** k, 1.75 * 2.0 ** k]
    rng = np.random.default_rng(0)
    vals += list(np.abs(rng.standard_normal(300)) * 2.0 ** rng.integers(-60, 60, 300))
    vals += [float(np.float32(v)) for v in rng.uniform(0, 1, 50) * 2.0 ** 126]
    got = oracle.mx_exponent(np.array(vals))
    exp = np.array([_exponent_search(v) for v in vals])
    assert np.array_equal(got, exp)


def _loop_quantise(x, axis):
    """Pure-Python loop over the blocks: the block's amax, its exponent by the
    exact search, then each element's e4m3 code of x * 2^-e."""
    x = x.double().numpy() if isinstance(x, torch.Tensor) else np.asarray(x, dtype=np.float64)
    B, H, N, d = x.shape
    codes = np.zeros((B, H, N, d), dtype=np.uint8)
    if axis == "rows":
        scales = np.zeros((B, H, N, d // ROW_BLOCK), dtype=np.uint8)
        blocks = [((b, h, n), [(n, c) for c in range(blk * ROW_BLOCK, (blk + 1) * ROW_BLOCK)], blk)
                  for b in range(B) for h in range(H) for n in range(N) for blk in range(d // ROW_BLOCK)]
    else:
        nb = -(-N // KEY_BLOCK)
        scales = np.zeros((B, H, nb, d), dtype=np.uint8)
        blocks = [((b, h, blk), [(n, c) for n in range(blk * KEY_BLOCK, min(N, (blk + 1) * KEY_BLOCK))], c)
                  for b in range(B) for h in range(H) for blk in range(nb) for c in range(d)]
    for (b, h, r), members, idx in blocks:
        amax = max(abs(x[b, h, n, c]) for n, c in members)
        e = _exponent_search(amax)
        scales[b, h, r, idx] = e + 127
        for n, c in members:
            codes[b, h, n, c] = oracle.e4m3_encode(np.array(x[b, h, n, c] * 2.0 ** -e))
    return codes, scales


def _inputs(N=37, d=64, seed=1):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((1, 2, N, d), generator=g)
    x[0, 0, 3, 5] = 900.0                       # an outlier
    x[0, 1, 10:20, :] *= 2.0 ** -20             # tiny rows
    x[0, 1, 30, :32] = 0.0                      # an all-zero row block
    x[0, 0, 33:, 7] = 0.0                       # an all-zero (ragged) key block
    return x.to(torch.bfloat16)


@pytest.mark.parametrize("axis", ["rows", "keys"])
def test_matches_the_block_loop(axis):
    x = _inputs()
    c, s = oracle.quantize_mx(x, axis)
    lc, ls = _loop_quantise(x, axis)
    assert np.array_equal(s, ls) and np.array_equal(c, lc)
    assert s.shape == ((1, 2, 37, 2) if axis == "rows" else (1, 2, 2, 64))


@pytest.mark.parametrize("axis", ["rows", "keys"])
def test_no_saturation_and_block_max_in_top_binades(axis):
    g = torch.Generator().manual_seed(2)
    x = (torch.randn((2, 3, 100, 128), generator=g) * 2.0 ** torch.randint(-30, 30, (2, 3, 100, 1), generator=g))
    x = x.to(torch.bfloat16)
    c, s = oracle.quantize_mx(x, axis)
    vals = np.abs(E4M3_VALUES[c])
    assert np.all(vals <= 448.0)

    def block_max(a):
        if axis == "rows":
            return a.reshape(2, 3, 100, 4, 32).max(-1)
        pad = np.zeros((2, 3, 128, 128))
        pad[:, :, :100] = a
        return pad.reshape(2, 3, 4, 32, 128).max(3)

    # before rounding the block's largest magnitude lies in (224, 448]; e4m3
    # rounding can take it down to 224 itself
    e = s.astype(np.float64) - 127
    scaled = block_max(np.abs(x.double().numpy())) * np.exp2(-e)
    assert np.all((scaled > 224.0) & (scaled <= 448.0))
    bmax = block_max(vals)
    assert np.all((bmax >= 224.0) & (bmax <= 448.0))


@pytest.mark.parametrize("axis", ["rows", "keys"])
def test_error_within_half_a_spacing(axis):
    x = _inputs(N=70, d=128, seed=3)
    c, s = oracle.quantize_mx(x, axis)
    xd = x.double().numpy()
    deq = oracle.dequantize_mx(c, s, axis)
    e = s.astype(np.int64) - 127
    e_el = np.repeat(e, 32, axis=-1) if axis == "rows" else np.repeat(e, 32, axis=2)[:, :, :70]
    # normal e4m3: spacing 2^-3 of the binade -> error <= 2^-4 |x|; subnormal: 2^(e-10)
    bound = np.maximum(2.0 ** -4 * np.abs(xd), np.ldexp(1.0, e_el - 10))
    assert np.all(np.abs(deq - xd) <= bound)


def test_representable_values_round_trip():
    rng = np.random.default_rng(4)
    codes = rng.integers(0, 0x7F, (1, 1, 64, 64)) | rng.integers(0, 2, (1, 1, 64, 64)) * 0x80
    codes[..., ::32] = 0x7E                     # every row block and key block holds 448
    e = rng.integers(-20, 20, (1, 1, 64, 2))
    x = E4M3_VALUES[codes] * np.exp2(np.repeat(e, 32, axis=-1))
    c, s = oracle.quantize_mx(x, "rows")
    assert np.array_equal(oracle.dequantize_mx(c, s, "rows"), x)
    assert np.array_equal(s.astype(np.int64) - 127, e)


def test_an_outlier_only_affects_its_own_block():
    x = _inputs(N=64, d=64, seed=5).double()
    y = x.clone()
    y[0, 0, 40, 3] = 3000.0
    for axis, changed in (("rows", (0, 0, 40, 0)), ("keys", (0, 0, 1, 3))):
        cx, sx = oracle.quantize_mx(x, axis)
        cy, sy = oracle.quantize_mx(y, axis)
        diff_s = np.argwhere(sx != sy)
        assert [tuple(r) for r in diff_s] == [changed]
        mask = np.ones(cx.shape, bool)
        if axis == "rows":
            mask[0, 0, 40, 0:32] = False
        else:
            mask[0, 0, 32:64, 3] = False
        assert np.array_equal(cx[mask], cy[mask])
    # one scale per head: the outlier changes the code of most values of its head
    cx, _ = oracle.quantize_per_head(x)
    cy, _ = oracle.quantize_per_head(y)
    assert np.count_nonzero(cx[0, 0] != cy[0, 0]) > 0.5 * cx[0, 0].size


def test_near_zero_majority_keeps_its_precision():
    # the failure mode: values huddle near zero with a few outliers far out
    g = torch.Generator().manual_seed(6)
    x = torch.randn((1, 1, 256, 128), generator=g) * 2.0 ** -10
    out = torch.rand(x.shape, generator=g) < 1.0 / 512
    x[out] = 64.0
    x = x.to(torch.bfloat16)
    xd = x.double().numpy()
    small = ~out.numpy() & (xd != 0)
    rel = lambda a: np.median(np.abs(a[small] - xd[small]) / np.abs(xd[small]))
    per_head = oracle.dequantize_per_head(*oracle.quantize_per_head(x))
    per_block = oracle.dequantize_mx(*oracle.quantize_mx(x, "rows"), "rows")
    assert rel(per_block) <= 2.0 ** -5          # e4m3's own rounding
    assert rel(per_head) >= 3 * rel(per_block)


def test_attention_on_dequantised_blocks_is_close():
    q, k, v = (_inputs(N=96, d=128, seed=s) for s in (7, 8, 9))
    (q8, qs), (k8, ks), (v8, vs) = oracle.quantize_qkv_mx(q, k, v)
    O, _ = oracle.attention(q, k, v, 1 / math.sqrt(128))
    Om, _ = oracle.attention(oracle.dequantize_mx(q8, qs, "rows"), oracle.dequantize_mx(k8, ks, "rows"),
                             oracle.dequantize_mx(v8, vs, "keys"), 1 / math.sqrt(128))
    a, b = Om.ravel(), O.ravel()
    assert a @ b / (np.linalg.norm(a) * np.linalg.norm(b)) > 0.999


def test_rotated_blocks_restore_the_scores():
    # rotated Q (1/d folded in) times rotated K^T gives back Q K^T; the fold is
    # exactly a factor 1/d on the values (a power of two moves only exponents)
    g = torch.Generator().manual_seed(12)
    q = torch.randn((1, 2, 50, 128), generator=g).to(torch.bfloat16)
    k = torch.randn((1, 2, 50, 128), generator=g).to(torch.bfloat16)
    q[..., 9] *= 30.0
    s = (1 - 2 * torch.randint(0, 2, (128,), generator=g)).numpy()
    qd = oracle.dequantize_mx(*oracle.quantize_rotated_mx(q, s, True), "rows")
    kd = oracle.dequantize_mx(*oracle.quantize_rotated_mx(k, s, False), "rows")
    S = np.einsum("bhnd,bhmd->bhnm", qd, kd)
    S_ref = np.einsum("bhnd,bhmd->bhnm", q.double().numpy(), k.double().numpy())
    assert np.corrcoef(S.ravel(), S_ref.ravel())[0, 1] > 0.999
    assert np.max(np.abs(S - S_ref)) < 0.1 * np.max(np.abs(S_ref))
    q_nofold = oracle.dequantize_mx(*oracle.quantize_rotated_mx(q, s, False), "rows")
    assert np.array_equal(qd * 128, q_nofold)


# --------------------------------------------------------------------------
# planted mistakes
# --------------------------------------------------------------------------
def _mutant(kind):
    def quantise(x, axis):
        xd = x.double().numpy() if isinstance(x, torch.Tensor) else np.asarray(x, dtype=np.float64)
        B, H, N, d = xd.shape
        if axis == "rows":
            blocks = xd.reshape(B, H, N, d // 32, 32)
        else:
            if kind == "keys_as_rows":
                blocks = xd.reshape(B, H, N, d // 32, 32)
            else:
                nb = -(-N // 32)
                pad = np.zeros((B, H, nb * 32, d))
                pad[:, :, :N] = xd
                blocks = np.moveaxis(pad.reshape(B, H, nb, 32, d), 3, -1)
        amax = np.abs(blocks).max(-1)
        with np.errstate(divide="ignore"):
            if kind == "ocp_floor":
                e = np.floor(np.log2(np.where(amax > 0, amax, 1.0))).astype(np.int64) - 8
            else:
                e = oracle.mx_exponent(amax) + (1 if kind == "one_too_high" else 0)
        scaled = np.ldexp(blocks, -e[..., None])
        if kind == "truncate":
            idx = np.searchsorted(E4M3_VALUES[:0x7F], np.abs(scaled), side="right") - 1
            codes = (np.clip(idx, 0, 0x7E) | np.where(np.signbit(scaled), 0x80, 0)).astype(np.uint8)
        else:
            codes = oracle.e4m3_encode(np.clip(scaled, -448, 448))
        if axis == "rows" or kind == "keys_as_rows":
            return codes.reshape(B, H, N, d), (e + 127).astype(np.uint8)
        codes = np.moveaxis(codes, -1, 3).reshape(B, H, -1, d)[:, :, :N]
        return codes, (e + 127).astype(np.uint8)
    return quantise


def _pins_pass(fn) -> bool:
    try:
        x = _inputs(N=70, d=64, seed=11)
        for axis in ("rows", "keys"):
            c, s = fn(x, axis)
            lc, ls = _loop_quantise(x, axis)
            if c.shape != lc.shape or s.shape != ls.shape:
                return False
            if not (np.array_equal(c, lc) and np.array_equal(s, ls)):
                return False
        return True
    except Exception:
        return False


def test_pins_accept_the_oracle():
    assert _pins_pass(oracle.quantize_mx)
    assert _pins_pass(_mutant("none"))


@pytest.mark.parametrize("kind", ["ocp_floor", "one_too_high", "truncate", "keys_as_rows"])
def test_pins_reject_planted_mistake(kind):
    assert not _pins_pass(_mutant(kind))
