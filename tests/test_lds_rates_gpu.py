"""LDS read throughput of the attention kernels' read patterns on one MI355X
CU (tests/hip/lds_rates.hip): what a wave's operand reads cost at the
backward's one wave per SIMD and at the forward's occupancy.

Patterns (32-row tiles of 256-byte bf16 rows, 16-byte chunks XOR-swizzled):
  * row-major ds_read_b128: lane = row l32, logical chunk 2u + hh, swizzle
    (row & 7) -- the K rows of the forward, the Q / dO rows of the backward;
  * transposed ds_read_b64_tr_b16 with the backward's swizzle (row & 7) and
    with the forward's V swizzle 2 (row & 3);
  * contiguous baselines.
Checked (printed in full): the swizzled row-major read runs at the speed of
a contiguous one; a transposed read of 512 bytes costs a wave at least as
long as a 1 KB row-major read, i.e. twice as long per byte; and, for the two
patterns the kernels use, one wave alone sees the same per-read time as one
wave on each of the four SIMDs, so the limit is each SIMD's read rate rather
than the shared LDS. Each rate is the fastest of three runs.
"""
import ctypes
import os

import pytest
import torch

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(__file__), "hip", "liblds_rates.so")
ROW = 256


def _rm(u):
    return [(l % 32) * ROW + 16 * (((2 * u + l // 32) ^ ((l % 32) & 7)) & 15) for l in range(64)]


def _tr(swz, t=0, n=0):
    out = []
    for l in range(64):
        vg, vj = l >> 4, l & 15
        va, hh, e, q = vg & 1, l >> 5, vj >> 2, vj & 3
        r = 4 * hh + e + 8 * t + 16 * n
        c = 2 * va + (q >> 1)
        out.append(r * ROW + 16 * ((c ^ swz(r)) & 15) + 8 * (q & 1))
    return out


def _run(lib, kind, offs, waves, trips=2000, repeats=3):
    """Cycles per read per wave: the fastest of `repeats` runs (anything else
    on the CU only ever slows a run down)."""
    assert len(offs) == 64 and all(0 <= o and o + 15 * 2048 + 16 <= 65536 for o in offs)
    assert all(o % (16 if kind == 0 else 8) == 0 for o in offs)
    o = torch.tensor(offs, dtype=torch.int32, device="cuda")
    sink = torch.zeros(64 * waves, dtype=torch.int32, device="cuda")
    cyc = torch.zeros(1, dtype=torch.int64, device="cuda")
    best = None
    for _ in range(repeats):
        assert lib.lds_rate_run(kind, o.data_ptr(), sink.data_ptr(), cyc.data_ptr(), trips, 64 * waves) == 0
        c = cyc.item() / (trips * 16)
        best = c if best is None else min(best, c)
    return best


def test_lds_read_rates():
    lib = ctypes.CDLL(LIB)
    lib.lds_rate_run.argtypes = [ctypes.c_int] + [ctypes.c_void_p] * 3 + [ctypes.c_int, ctypes.c_int]
    res = {}
    for waves in (1, 4, 16):
        res[("b128 contiguous", waves)] = _run(lib, 0, [16 * l for l in range(64)], waves)
        res[("b128 rows, swizzle row&7", waves)] = max(_run(lib, 0, _rm(u), waves) for u in range(4))
        res[("tr16 rows, swizzle row&7", waves)] = max(_run(lib, 1, _tr(lambda r: r & 7, t, n), waves)
                                                       for t in (0, 1) for n in (0, 1))
        res[("tr16 rows, swizzle 2(row&3)", waves)] = max(_run(lib, 1, _tr(lambda r: 2 * (r & 3), t, n), waves)
                                                          for t in (0, 1) for n in (0, 1))
    for (name, waves), c in res.items():
        nbytes = 1024 if name.startswith("b128") else 512
        print(f"{name:30s} {waves:2d} wave(s): {c:6.1f} cycles per read per wave, "
              f"{waves * nbytes / c:6.1f} B/cycle for the CU", flush=True)
    assert res[("b128 rows, swizzle row&7", 1)] <= 1.10 * res[("b128 contiguous", 1)]
    assert res[("tr16 rows, swizzle row&7", 1)] >= 1.0 * res[("b128 contiguous", 1)]
    # the per-SIMD claim, on the two patterns the kernels read with
    for name in ("b128 rows, swizzle row&7", "tr16 rows, swizzle row&7"):
        assert res[(name, 4)] <= 1.25 * res[(name, 1)]
