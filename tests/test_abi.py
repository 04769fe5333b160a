"""The C ABI loads, exports every symbol include/fa.h declares, and rejects bad
arguments with the documented status codes before anything is launched. No
compute call is made here, so these run without a GPU."""
import ctypes
import os
import re
import subprocess

import pytest

from tiled_attention_fa2_amd import fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


def _header_text():
    return open(HEADER).read()


def _declared_functions():
    txt = re.sub(r"/\*.*?\*/", "", _header_text(), flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", txt)))


def _header_enum(name_prefix):
    txt = _header_text()
    return {m.group(1): int(m.group(2)) for m in re.finditer(rf"\b({name_prefix}[A-Z0-9_]*)\s*=\s*(-?\d+)", txt)}


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.LIB_PATH):
        pytest.skip("libfa.so not built")
    return fa.lib()


def test_header_declares_expected_entry_points():
    assert _declared_functions() == ["fa_bwd", "fa_bwd_workspace_bytes", "fa_fwd", "fa_fwd_gqa",
                                     "fa_fwd_mxfp8", "fa_fwd_splitkv", "fa_fwd_splitkv_static", "fa_merge_partials", "fa_quantize_fp8", "fa_quantize_fp8_rotated",
                                     "fa_quantize_mxfp8_keys", "fa_quantize_mxfp8_rows",
                                     "fa_splitkv_chunk_keys", "fa_splitkv_default_splits",
                                     "fa_splitkv_workspace_bytes", "fa_status_string"]


def test_every_declared_symbol_is_exported(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", fa.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (fa_[a-z0-9_]+)\b", out))
    assert set(_declared_functions()) <= exported


def test_binding_constants_match_header():
    dt = _header_enum("FA_DTYPE_")
    assert dt == {"FA_DTYPE_F32": fa.DTYPE_F32, "FA_DTYPE_BF16": fa.DTYPE_BF16,
                  "FA_DTYPE_FP8_E4M3": fa.DTYPE_FP8_E4M3}
    st = {v: k for k, v in _header_enum("FA_").items() if not k.startswith("FA_DTYPE_")}
    assert st == fa.STATUS
    m = re.search(r"#define\s+FA_MAX_SPLITS\s+(\d+)", _header_text())
    assert m and int(m.group(1)) == fa.FA_MAX_SPLITS
    m = re.search(r"#define\s+FA_STATIC_SCRATCH_BYTES\s+\((\d+)u\s*<<\s*(\d+)\)", _header_text())
    assert m and int(m.group(1)) << int(m.group(2)) == fa.STATIC_SCRATCH_BYTES


def test_status_strings(lib):
    for code, name in fa.STATUS.items():
        assert fa.status_string(code).startswith(name)
    assert fa.status_string(12345) == "unknown fa status"


# pointers that are never dereferenced: validation returns first
A = ctypes.c_void_p(0x10000)
A2 = ctypes.c_void_p(0x20000)
MIS = ctypes.c_void_p(0x10008)


def _fwd(lib, q=A, k=A, v=A, o=A2, lse=A2, B=1, H=1, N=128, d=128, causal=0, scale=0.1,
         dtype=1, descales=None):
    return lib.fa_fwd(q, k, v, o, lse, B, H, N, d, causal, scale, dtype, descales, None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), -2), (dict(H=-3), -2), (dict(N=-1), -2),
    (dict(dtype=7), -3), (dict(dtype=-1), -3),
    (dict(d=96), -4), (dict(d=256), -4), (dict(d=0), -4),
    (dict(scale=float("nan")), -5), (dict(scale=float("inf")), -5),
    (dict(dtype=2, descales=None), -6),
    (dict(q=None), -1), (dict(o=None), -1), (dict(lse=None), -1),
    (dict(q=MIS), -7), (dict(v=MIS), -7), (dict(o=MIS), -7),
    (dict(N=0), 0), (dict(B=0), 0), (dict(H=0), 0),
    (dict(B=1 << 20, H=1 << 12, N=4096), -2),
    # one head is addressed with 32-bit byte offsets: (N + 128) * d * bytes per
    # element must not exceed INT_MAX (a tile may read up to 128 rows past N)
    (dict(N=(1 << 31) // 256 - 128), -2),                           # bf16, d = 128: 2^31 bytes
    (dict(N=(1 << 31) // 128 - 128, dtype=2, descales=A2), -2),     # fp8, d = 128
    (dict(N=(1 << 31) // 256 - 128, d=64, dtype=0), -2),            # fp32, d = 64
])
def test_fwd_validation_codes(lib, kw, code):
    assert _fwd(lib, **kw) == code


@pytest.mark.parametrize("args,code", [
    ((A, 1, A2, A2, -1, 1, 16, 64), -2),
    ((A, 2, A2, A2, 1, 1, 16, 64), -3),
    ((A, 1, A2, A2, 1, 1, 16, 32), -4),
    ((A, 1, A2, None, 1, 1, 16, 64), -1),
    ((None, 1, A2, A2, 1, 1, 16, 64), -1),
    ((MIS, 1, A2, A2, 1, 1, 16, 64), -7),
    ((A, 1, A2, A2, 0, 4, 16, 64), 0),
    ((A, 1, A2, A2, 1, 1 << 17, 16, 64), -2),
])
def test_quantize_validation_codes(lib, args, code):
    assert lib.fa_quantize_fp8(*args, None) == code


# (x, in_dtype, signs, x_fp8, descale, B, H, N, d, fold)
@pytest.mark.parametrize("args,code", [
    ((A, 1, A, A2, A2, -1, 1, 16, 64, 1), -2),
    ((A, 0, A, A2, A2, 1, 1, 16, 64, 1), -3),       # float32 input is not taken
    ((A, 2, A, A2, A2, 1, 1, 16, 64, 1), -3),
    ((A, 1, A, A2, A2, 1, 1, 16, 32, 0), -4),
    ((A, 1, A, A2, A2, 1, 1, 16, 96, 0), -4),
    ((A, 1, None, A2, A2, 1, 1, 16, 64, 0), -1),
    ((A, 1, A, A2, None, 1, 1, 16, 64, 0), -1),
    ((None, 1, A, A2, A2, 1, 1, 16, 64, 0), -1),
    ((A, 1, A, None, A2, 1, 1, 16, 64, 0), -1),
    ((MIS, 1, A, A2, A2, 1, 1, 16, 64, 0), -7),
    ((A, 1, A, MIS, A2, 1, 1, 16, 64, 0), -7),
    ((A, 1, A, A2, A2, 0, 4, 16, 64, 1), 0),
    ((A, 1, A, A2, A2, 1, 1 << 17, 16, 64, 1), -2),
])
def test_quantize_rotated_validation_codes(lib, args, code):
    assert lib.fa_quantize_fp8_rotated(*args, None) == code


# (x, in_dtype, signs, fold, x_fp8, scales, B, H, N, d)
@pytest.mark.parametrize("args,code", [
    ((A, 1, None, 0, A2, A2, -1, 1, 16, 64), -2),
    ((A, 2, None, 0, A2, A2, 1, 1, 16, 64), -3),
    ((A, 0, A, 0, A2, A2, 1, 1, 16, 64), -3),        # rotation needs bfloat16
    ((A, 1, None, 0, A2, A2, 1, 1, 16, 96), -4),
    ((None, 1, None, 0, A2, A2, 1, 1, 16, 64), -1),
    ((A, 1, None, 0, None, A2, 1, 1, 16, 64), -1),
    ((A, 1, None, 0, A2, None, 1, 1, 16, 64), -1),
    ((MIS, 1, None, 0, A2, A2, 1, 1, 16, 64), -7),
    ((A, 1, None, 0, MIS, A2, 1, 1, 16, 64), -7),
    ((A, 1, None, 0, A2, A2, 0, 4, 16, 64), 0),
    ((A, 1, None, 0, A2, A2, 1, 1, 0, 64), 0),
    ((A, 1, A, 1, A2, A2, 1, 1 << 17, 16, 64), -2),
])
def test_quantize_mxfp8_rows_validation_codes(lib, args, code):
    assert lib.fa_quantize_mxfp8_rows(*args, None) == code


# (x, in_dtype, x_fp8, scales, B, H, N, d)
@pytest.mark.parametrize("args,code", [
    ((A, 1, A2, A2, -1, 1, 16, 64), -2),
    ((A, 7, A2, A2, 1, 1, 16, 64), -3),
    ((A, 1, A2, A2, 1, 1, 16, 32), -4),
    ((A, 1, None, A2, 1, 1, 16, 64), -1),
    ((A, 1, A2, None, 1, 1, 16, 64), -1),
    ((MIS, 1, A2, A2, 1, 1, 16, 64), -7),
    ((A, 1, A2, ctypes.c_void_p(0x20002), 1, 1, 16, 64), -7),
    ((A, 1, A2, A2, 1, 0, 16, 64), 0),
])
def test_quantize_mxfp8_keys_validation_codes(lib, args, code):
    assert lib.fa_quantize_mxfp8_keys(*args, None) == code


def _fwd_mx(lib, q=A, k=A, v=A, qs=A2, ks=A2, vs=A2, o=A2, lse=A2, B=1, Hq=2, Hkv=1, N=128, d=128, causal=0,
            scale=0.1, splits=1, ws=None, wsb=0):
    return lib.fa_fwd_mxfp8(q, k, v, qs, ks, vs, o, lse, B, Hq, Hkv, N, d, causal, scale, splits, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), -2), (dict(Hkv=3), -2), (dict(d=64), -4), (dict(d=96), -4),
    (dict(scale=float("nan")), -5), (dict(qs=None), -6), (dict(vs=None), -6),
    (dict(q=None), -1), (dict(q=MIS), -7), (dict(ks=ctypes.c_void_p(0x20001)), -7),
    (dict(splits=0), -10), (dict(splits=65), -10), (dict(splits=2), -9),
    (dict(N=0), 0), (dict(B=0), 0),
])
def test_fwd_mxfp8_validation_codes(lib, kw, code):
    assert _fwd_mx(lib, **kw) == code


def test_binding_raises_when_library_missing(monkeypatch, tmp_path):
    monkeypatch.setattr(fa, "LIB_PATH", str(tmp_path / "absent.so"))
    monkeypatch.setattr(fa, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        fa.lib()


# --------------------------------------------------------------------------
# split-KV: host-side helpers and validation (nothing is launched)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("N,S,chunk", [
    (4096, 1, 4096), (4096, 3, 1408), (4096, 4, 1024), (30272, 3, 10112),
    (200, 4, 128), (1, 1, 128), (129, 2, 128), (0, 2, 0), (100, 0, 0), (100, 65, 0),
])
def test_chunk_keys(lib, N, S, chunk):
    # 128 * ceil(ceil(N / S) / 128)
    assert lib.fa_splitkv_chunk_keys(N, S) == chunk


def test_workspace_bytes(lib):
    assert fa.splitkv_workspace_bytes(1, 8, 4096, 128, 3) == 4 * 3 * 8 * 4096 * 129
    assert fa.splitkv_workspace_bytes(2, 3, 100, 64, 5) == 4 * 5 * 6 * 100 * 65
    assert fa.splitkv_workspace_bytes(1, 1, 100, 96, 2) == 0
    assert fa.splitkv_workspace_bytes(1, 1, 100, 64, 0) == 0
    assert fa.splitkv_workspace_bytes(-1, 1, 100, 64, 2) == 0


def test_default_splits_is_at_least_one(lib):
    for args in [(1, 8, 4096, 128, 0, 1), (1, 56, 30272, 128, 0, 1), (0, 1, 1, 64, 0, 0),
                 (1, 1, 100, 96, 0, 1)]:
        assert lib.fa_splitkv_default_splits(*args) >= 1


WS = ctypes.c_void_p(0x40000)


def _split(lib, num_splits=2, ws=WS, ws_bytes=1 << 40, **kw):
    p = dict(q=A, k=A, v=A, o=A2, lse=A2, B=1, H=1, N=128, d=128, causal=0, scale=0.1, dtype=1,
             descales=None)
    p.update(kw)
    return lib.fa_fwd_splitkv(p["q"], p["k"], p["v"], p["o"], p["lse"], p["B"], p["H"], p["N"],
                              p["d"], p["causal"], p["scale"], p["dtype"], p["descales"], num_splits,
                              ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), -2), (dict(dtype=5), -3), (dict(d=32), -4), (dict(scale=float("nan")), -5),
    (dict(dtype=2), -6), (dict(q=None), -1), (dict(k=MIS), -7),
    (dict(num_splits=0), -10), (dict(num_splits=65), -10), (dict(num_splits=-2), -10),
    (dict(ws=None), -9), (dict(ws=ctypes.c_void_p(0x40004)), -9),
    (dict(ws_bytes=4 * 2 * 128 * 129 - 1), -9),
    (dict(N=0), 0), (dict(H=0), 0),
])
def test_splitkv_validation_codes(lib, kw, code):
    assert _split(lib, **kw) == code


def _split_static(lib, num_splits=2, **kw):
    p = dict(q=A, k=A, v=A, o=A2, lse=A2, B=1, H=1, N=128, d=128, causal=0, scale=0.1, dtype=1,
             descales=None)
    p.update(kw)
    return lib.fa_fwd_splitkv_static(p["q"], p["k"], p["v"], p["o"], p["lse"], p["B"], p["H"], p["N"],
                                     p["d"], p["causal"], p["scale"], p["dtype"], p["descales"],
                                     num_splits, None)


# the partials of B*H*N rows in S chunks take 4*S*B*H*N*(d+1) bytes; 64 MiB holds
# 8 heads of 4096 tokens in 3 chunks (50.7 MB) but not in 4 (67.6 MB)
@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), -2), (dict(dtype=5), -3), (dict(d=32), -4), (dict(scale=float("nan")), -5),
    (dict(dtype=2), -6), (dict(q=None), -1), (dict(k=MIS), -7), (dict(o=MIS), -7),
    (dict(num_splits=0), -10), (dict(num_splits=65), -10), (dict(num_splits=-1), -10),
    (dict(N=0), 0), (dict(H=0), 0), (dict(num_splits=0, N=0), -10),
    (dict(H=8, N=4096, num_splits=4), -11),
    (dict(H=56, N=30272, num_splits=2), -11),
    (dict(B=1 << 20, H=1 << 12, N=4096), -2),
])
def test_splitkv_static_validation_codes(lib, kw, code):
    assert _split_static(lib, **kw) == code


def test_static_scratch_limit_is_the_documented_size(lib):
    # the largest accepted problem needs at most FA_STATIC_SCRATCH_BYTES
    assert lib.fa_splitkv_workspace_bytes(1, 8, 4096, 128, 3) <= fa.STATIC_SCRATCH_BYTES
    assert lib.fa_splitkv_workspace_bytes(1, 8, 4096, 128, 4) > fa.STATIC_SCRATCH_BYTES


def _merge(lib, op=A, lp=A2, S=2, B=1, H=1, N=16, d=128, out_dtype=1, o=WS, lse=A2):
    return lib.fa_merge_partials(op, lp, S, B, H, N, d, out_dtype, o, lse, None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), -2), (dict(out_dtype=2), -3), (dict(out_dtype=9), -3), (dict(d=96), -4),
    (dict(S=0), -10), (dict(S=65), -10),
    (dict(op=None), -1), (dict(lp=None), -1), (dict(o=None), -1), (dict(lse=None), -1),
    (dict(op=MIS), -7), (dict(o=MIS), -7),
    (dict(N=0), 0), (dict(B=0), 0),
])
def test_merge_validation_codes(lib, kw, code):
    assert _merge(lib, **kw) == code


def _gqa(lib, Hq=8, Hkv=2, num_splits=1, ws=None, ws_bytes=0, **kw):
    p = dict(q=A, k=A, v=A, o=A2, lse=A2, B=1, N=128, d=128, causal=0, scale=0.1, dtype=1, descales=None)
    p.update(kw)
    return lib.fa_fwd_gqa(p["q"], p["k"], p["v"], p["o"], p["lse"], p["B"], Hq, Hkv, p["N"], p["d"],
                          p["causal"], p["scale"], p["dtype"], p["descales"], num_splits, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(Hq=6, Hkv=4), -2), (dict(Hkv=0), -2), (dict(Hkv=-2), -2), (dict(Hq=-1), -2), (dict(N=-3), -2),
    (dict(dtype=4), -3), (dict(d=80), -4), (dict(scale=float("inf")), -5), (dict(dtype=2), -6),
    (dict(v=None), -1), (dict(o=MIS), -7),
    (dict(num_splits=0), -10), (dict(num_splits=65), -10),
    (dict(num_splits=2), -9), (dict(num_splits=2, ws=ctypes.c_void_p(0x40008), ws_bytes=1 << 40), -9),
    (dict(num_splits=3, ws=WS, ws_bytes=4 * 3 * 8 * 128 * 129 - 4), -9),
    (dict(B=0), 0), (dict(N=0), 0), (dict(B=0, num_splits=4), 0),
])
def test_gqa_validation_codes(lib, kw, code):
    assert _gqa(lib, **kw) == code


def _bwd(lib, Hq=2, Hkv=2, ws=WS, ws_bytes=1 << 40, **kw):
    p = dict(q=A, k=A, v=A, o=A, do=A, lse=A2, dq=A2, dk=A2, dv=A2, B=1, N=128, d=128, causal=0,
             scale=0.1, dtype=1)
    p.update(kw)
    return lib.fa_bwd(p["q"], p["k"], p["v"], p["o"], p["do"], p["lse"], p["dq"], p["dk"], p["dv"],
                      p["B"], Hq, Hkv, p["N"], p["d"], p["causal"], p["scale"], p["dtype"], ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), -2), (dict(Hq=4, Hkv=3), -2), (dict(Hkv=0), -2),
    (dict(dtype=0), -3), (dict(dtype=2), -3), (dict(d=96), -4), (dict(scale=float("nan")), -5),
    (dict(o=None), -1), (dict(do=None), -1), (dict(lse=None), -1), (dict(dk=None), -1),
    (dict(dq=MIS), -7), (dict(do=MIS), -7),
    (dict(ws=None), -9), (dict(ws=ctypes.c_void_p(0x40004)), -9), (dict(ws_bytes=8 * 2 * 128 - 1), -9),
    (dict(N=0), 0), (dict(B=0), 0),
])
def test_bwd_validation_codes(lib, kw, code):
    assert _bwd(lib, **kw) == code


def test_bwd_workspace_bytes(lib):
    assert fa.bwd_workspace_bytes(2, 3, 100) == 8 * 2 * 3 * 100
    assert fa.bwd_workspace_bytes(-1, 3, 100) == 0


def test_binding_rejects_host_tensors_before_any_launch():
    import torch

    x = torch.zeros((1, 1, 4, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.quantize_fp8(x)
    with pytest.raises(ValueError):
        fa.fwd(x, x, x)
    assert fa._device(None, None) is None
    with pytest.raises(ValueError, match="device tensor"):
        fa._device(None, x)
