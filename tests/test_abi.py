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
    assert _declared_functions() == ["fa_fwd", "fa_quantize_fp8", "fa_status_string"]


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


def test_binding_raises_when_library_missing(monkeypatch, tmp_path):
    monkeypatch.setattr(fa, "LIB_PATH", str(tmp_path / "absent.so"))
    monkeypatch.setattr(fa, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        fa.lib()
