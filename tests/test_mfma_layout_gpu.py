"""The MFMA lane layouts the attention kernel is built on, checked on the
hardware with a one-wave probe (tests/hip/mfma_probe.hip), and the
accumulation precision of the fp8 MFMA.

Layouts assumed by the kernel (32x32 MFMAs, K = 2, 16 or 64):
  A[i][k]: lane i + 32*(k // KPL), slot k % KPL      (KPL = K / 2)
  B[k][j]: lane j + 32*(k // KPL), slot k % KPL
  D[i][j]: lane j + 32*((i // 4) % 2), register 4*(i // 8) + i % 4
For the fp8 MFMA only the pairing of slots matters (the kernel fills A and B
through the same mapping), so the check there is that lane-half h slot s of A
meets lane-half h slot s of B, with D in the layout above.
"""
import ctypes
import os

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(__file__), "hip", "libmfma_probe.so")

# Bound on |fp8 MFMA result - exact sum| relative to sum |a_k b_k| over the
# products of one MFMA, used by the fp8 stress tests. The probe below checks
# the hardware stays within it.
EPS_FP8_ACC = 2.0 ** -10


def _probe(kind, a, b):
    lib = ctypes.CDLL(LIB)
    lib.probe_mfma.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    c = torch.zeros(64 * 16, dtype=torch.float32, device="cuda")
    assert lib.probe_mfma(kind, a.data_ptr(), b.data_ptr(), c.data_ptr()) == 0
    return c.cpu().numpy().reshape(64, 16)


def _expected(Amat, Bmat):
    D = Amat @ Bmat
    return np.array([[D[8 * (r // 4) + 4 * (l // 32) + r % 4, l % 32] for r in range(16)]
                     for l in range(64)])


@pytest.mark.parametrize("kind,kpl", [(0, 1), (1, 8)])
def test_float_mfma_layouts(kind, kpl):
    rng = np.random.default_rng(kind)
    a = rng.integers(-3, 4, (64, kpl)).astype(np.float32)
    b = rng.integers(-3, 4, (64, kpl)).astype(np.float32)
    K = 2 * kpl
    A = np.zeros((32, K))
    B = np.zeros((K, 32))
    for l in range(64):
        for s in range(kpl):
            A[l % 32, (l // 32) * kpl + s] = a[l, s]
            B[(l // 32) * kpl + s, l % 32] = b[l, s]
    got = _probe(kind, torch.from_numpy(a.ravel()).cuda(), torch.from_numpy(b.ravel()).cuda())
    assert np.array_equal(got, _expected(A, B))


def _fp8_run(ac, bc):
    tab = oracle.e4m3_table()
    got = _probe(2, torch.from_numpy(ac.astype(np.uint8)).view(torch.int32).cuda(),
                 torch.from_numpy(bc.astype(np.uint8)).view(torch.int32).cuda())
    av = tab[ac.reshape(64, 32)]
    bv = tab[bc.reshape(64, 32)]
    # A[i][(h, s)] = lane i + 32h slot s; B[(h, s)][j] = lane j + 32h slot s
    A = np.concatenate([av[:32], av[32:]], axis=1)
    B = np.concatenate([bv[:32], bv[32:]], axis=1).T
    return got, _expected(A, B), _expected(np.abs(A), np.abs(B))


def test_fp8_mfma_pairing_exact_on_small_codes():
    rng = np.random.default_rng(3)
    sg = lambda: rng.integers(0, 2, 64 * 32) * 0x80
    ac = rng.integers(0x30, 0x40, 64 * 32) | sg()     # magnitudes 0.5 .. 1.9
    bc = rng.integers(0x30, 0x40, 64 * 32) | sg()
    got, exp, _ = _fp8_run(ac, bc)
    assert np.array_equal(got, exp)


def test_fp8_mfma_accumulation_precision():
    rng = np.random.default_rng(4)
    worst = 0.0
    for trial in range(8):
        ac = rng.integers(0, 0x7F, 64 * 32) | rng.integers(0, 2, 64 * 32) * 0x80
        bc = rng.integers(0, 0x7F, 64 * 32) | rng.integers(0, 2, 64 * 32) * 0x80
        got, exp, mag = _fp8_run(ac, bc)
        worst = max(worst, float(np.max(np.abs(got - exp) / np.maximum(mag, 1e-30))))
    one, big = 0x38, 0x7E
    ac = np.full(64 * 32, one)
    ac[0::32] = big
    got, exp, mag = _fp8_run(ac, ac.copy())
    worst = max(worst, float(np.max(np.abs(got - exp) / mag)))
    print(f"fp8 MFMA: max |err| / sum|a*b| = {worst:.3e} (2^{np.log2(max(worst, 1e-30)):.1f})")
    assert worst <= EPS_FP8_ACC


def _probe_scaled(variant, ac, bc, sa, sb):
    lib = ctypes.CDLL(LIB)
    lib.probe_mfma_scaled.argtypes = [ctypes.c_int] + [ctypes.c_void_p] * 5
    dev = [torch.from_numpy(np.ascontiguousarray(x)).cuda()
           for x in (ac.astype(np.uint8), bc.astype(np.uint8), sa.astype(np.uint32), sb.astype(np.uint32))]
    a, b, sa_d, sb_d = (t.view(torch.int32) for t in dev)
    c = torch.zeros(64 * 16, dtype=torch.float32, device="cuda")
    assert lib.probe_mfma_scaled(variant, a.data_ptr(), b.data_ptr(), sa_d.data_ptr(), sb_d.data_ptr(),
                                 c.data_ptr()) == 0
    return c.cpu().numpy().reshape(64, 16)


@pytest.mark.parametrize("variant,opa,opb", [(0, 0, 0), (1, 2, 1), (2, 3, 3)])
def test_fp8_scaled_mfma_per_lane_scales(variant, opa, opb):
    # The per-block FP8 path relies on this layout of the scaled fp8 MFMA
    # (32x32x64): lane half h slot s holds k = 32 (s // 16) + 16 h + s % 16, so
    # the contraction block b (k = 32b .. 32b + 31) is slots 16b .. 16b + 15
    # of both lane halves, and its E8M0 scale for row i of A (column j of B)
    # comes from lane i + 32b (j + 32b); opsel picks the byte of that lane's
    # scale register.
    rng = np.random.default_rng(10 + variant)
    sg = lambda: rng.integers(0, 2, 64 * 32) * 0x80
    ac = rng.integers(0x30, 0x40, 64 * 32) | sg()
    bc = rng.integers(0x30, 0x40, 64 * 32) | sg()
    # scales 2^-1 .. 2^1 keep every sum exact in fp32 (multiples of 2^-10 below 2^10)
    sa_bytes = rng.integers(126, 129, (64, 4))
    sb_bytes = rng.integers(126, 129, (64, 4))
    pack = lambda by: (by[:, 0] | (by[:, 1] << 8) | (by[:, 2] << 16) | (by[:, 3] << 24)).astype(np.uint32)
    got = _probe_scaled(variant, ac, bc, pack(sa_bytes), pack(sb_bytes))
    tab = oracle.e4m3_table()
    av, bv = tab[ac.reshape(64, 32)], tab[bc.reshape(64, 32)]
    A = np.zeros((32, 64))
    B = np.zeros((64, 32))
    for l in range(64):
        i, h = l % 32, l // 32
        for sl in range(32):
            blk = sl // 16
            k = 32 * blk + 16 * h + sl % 16
            A[i, k] = av[l, sl] * 2.0 ** (sa_bytes[i + 32 * blk, opa] - 127)
            B[k, i] = bv[l, sl] * 2.0 ** (sb_bytes[i + 32 * blk, opb] - 127)
    exp = _expected(A, B)
    print(f"max |got - expected| = {np.max(np.abs(got - exp)):.3e}, max |expected| = {np.max(np.abs(exp)):.3e}")
    assert np.array_equal(got, exp)
