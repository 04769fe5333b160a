"""Pins for the rotation-before-quantisation oracle (CPU only).

"Kernels and Memory in LLM Inference", section "Precision: FP8 with a real
failure mode": Q and K are multiplied by a fixed random rotation before FP8
quantisation; Q K^T is unchanged. Pinned here: the Sylvester construction
against the popcount formula of Hadamard matrices; H H^T = d I; rotated Q
times rotated K^T = d Q K^T; the fp32 result against an exact rational sum
(fractions) rounded once; the rotation of a basis vector is a signed row of
H; the folded 1/d; a large outlier coordinate spreads out; planted mistakes.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle


def _signs(d, seed):
    return np.where(np.random.default_rng(seed).integers(0, 2, d) == 1, 1.0, -1.0)


@pytest.mark.parametrize("d", [1, 2, 8, 64, 128])
def test_sylvester_matches_popcount_formula_and_is_orthogonal(d):
    H = oracle.hadamard(d)
    i, j = np.meshgrid(np.arange(d), np.arange(d), indexing="ij")
    pop = np.vectorize(lambda t: bin(t).count("1"))(i & j)
    assert np.array_equal(H, (-1.0) ** pop)
    assert np.array_equal(H @ H.T, d * np.eye(d))


def test_rejects_non_power_of_two():
    with pytest.raises(ValueError):
        oracle.hadamard(96)


def test_dot_products_scale_by_d():
    g = torch.Generator().manual_seed(0)
    q = torch.randn((3, 128), generator=g, dtype=torch.float64).numpy()
    k = torch.randn((5, 128), generator=g, dtype=torch.float64).numpy()
    s = _signs(128, 1)
    H = oracle.hadamard(128)
    qr, kr = (q * s) @ H, (k * s) @ H
    assert np.allclose(qr @ kr.T, 128 * (q @ k.T), atol=1e-9)


def test_fp32_values_are_the_exact_sums_rounded_once():
    g = torch.Generator().manual_seed(2)
    x = torch.randn((4, 64), generator=g).to(torch.bfloat16)
    s = _signs(64, 3)
    y = oracle.rotate(x, s)
    H = oracle.hadamard(64)
    xf = x.double().numpy()
    for r in range(4):
        for c in (0, 1, 17, 63):
            exact = sum(Fraction(float(xf[r, i])) * int(s[i]) * int(H[i, c]) for i in range(64))
            assert y[r, c] == np.float32(float(exact))


def test_basis_vector_gives_signed_hadamard_row():
    s = _signs(8, 4)
    for i in range(8):
        e = np.zeros(8)
        e[i] = 1.0
        assert np.array_equal(oracle.rotate(e, s), (s[i] * oracle.hadamard(8)[i]).astype(np.float32))


def test_outlier_coordinate_spreads():
    x = np.full((1, 128), 0.01)
    x[0, 5] = 50.0
    y = oracle.rotate(x, _signs(128, 5))
    # one loud coordinate becomes 128 of magnitude ~50: max/rms drops from ~11 to ~1
    assert np.max(np.abs(x)) / np.sqrt(np.mean(x ** 2)) > 10
    assert np.max(np.abs(y)) / np.sqrt(np.mean(y.astype(np.float64) ** 2)) < 1.1


def test_folded_descale_restores_the_scores():
    g = torch.Generator().manual_seed(6)
    q = torch.randn((1, 2, 40, 128), generator=g).to(torch.bfloat16)
    k = torch.randn((1, 2, 40, 128), generator=g).to(torch.bfloat16)
    s = _signs(128, 7)
    cq, dq = oracle.quantize_rotated(q, s, fold_inverse_d=True)
    ck, dk = oracle.quantize_rotated(k, s, fold_inverse_d=False)
    _, dq_plain = oracle.quantize_per_head(oracle.rotate(q, s))
    assert np.array_equal(dq, (dq_plain / np.float32(128)).astype(np.float32))
    qd = oracle.dequantize_per_head(cq, dq)
    kd = oracle.dequantize_per_head(ck, dk)
    S = np.einsum("bhnd,bhmd->bhnm", qd, kd)
    S_ref = np.einsum("bhnd,bhmd->bhnm", q.double().numpy(), k.double().numpy())
    # within the FP8 rounding of both operands
    assert np.max(np.abs(S - S_ref)) < 0.25 * np.max(np.abs(S_ref))
    assert np.corrcoef(S.ravel(), S_ref.ravel())[0, 1] > 0.999


@pytest.mark.parametrize("kind", ["normalised", "transposed_signs", "no_signs"])
def test_pins_reject_mistakes(kind):
    g = torch.Generator().manual_seed(8)
    x = torch.randn((2, 128), generator=g).to(torch.bfloat16)
    s = _signs(128, 9)
    H = oracle.hadamard(128)
    xf = x.double().numpy()
    if kind == "normalised":
        wrong = ((xf * s) @ H / math.sqrt(128)).astype(np.float32)
    elif kind == "transposed_signs":
        wrong = ((xf @ H) * s).astype(np.float32)
    else:
        wrong = (xf @ H).astype(np.float32)
    exact = np.array([[np.float32(float(sum(Fraction(float(xf[r, i])) * int(s[i]) * int(H[i, c])
                                            for i in range(128)))) for c in range(128)] for r in range(2)])
    assert np.array_equal(oracle.rotate(x, s), exact)
    assert not np.array_equal(wrong, exact)
