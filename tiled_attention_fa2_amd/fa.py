"""Python binding of libfa.so (argument marshalling only).

Every step of the attention forward and of the FP8 quantiser runs in the HIP
kernels behind the C ABI of include/fa.h. This module only checks tensor
metadata, allocates outputs with torch, and passes raw device pointers plus
torch's current HIP stream. There is no fallback: if libfa.so is missing or a
call fails, it raises.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfa.so")

# values of fa_dtype_t and fa_status_t in include/fa.h
DTYPE_F32, DTYPE_BF16, DTYPE_FP8_E4M3 = 0, 1, 2
FA_OK = 0
STATUS = {0: "FA_OK", -1: "FA_ERR_NULL", -2: "FA_ERR_SHAPE", -3: "FA_ERR_DTYPE",
          -4: "FA_ERR_HEAD_DIM", -5: "FA_ERR_SCALE", -6: "FA_ERR_DESCALES",
          -7: "FA_ERR_ALIGN", -8: "FA_ERR_HIP", -9: "FA_ERR_WORKSPACE", -10: "FA_ERR_SPLITS",
          -11: "FA_ERR_SCRATCH"}
FA_MAX_SPLITS = 64
STATIC_SCRATCH_BYTES = 64 << 20   # FA_STATIC_SCRATCH_BYTES

_lib = None


class FAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where} failed: {status_string(status)} ({status})")


def lib() -> ctypes.CDLL:
    """Load libfa.so once. Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing; build it with "
                               "`python -m tiled_attention_fa2_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        L.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, vp]
        L.fa_fwd.restype = i
        L.fa_quantize_fp8.argtypes = [vp, i, vp, vp, i, i, i, i, vp]
        L.fa_quantize_fp8.restype = i
        L.fa_quantize_fp8_rotated.argtypes = [vp, i, vp, vp, vp, i, i, i, i, i, vp]
        L.fa_quantize_fp8_rotated.restype = i
        L.fa_quantize_mxfp8_rows.argtypes = [vp, i, vp, i, vp, vp, i, i, i, i, vp]
        L.fa_quantize_mxfp8_rows.restype = i
        L.fa_quantize_mxfp8_keys.argtypes = [vp, i, vp, vp, i, i, i, i, vp]
        L.fa_quantize_mxfp8_keys.restype = i
        L.fa_status_string.argtypes = [i]
        L.fa_status_string.restype = ctypes.c_char_p
        sz = ctypes.c_size_t
        L.fa_splitkv_chunk_keys.argtypes = [i, i]
        L.fa_splitkv_chunk_keys.restype = i
        L.fa_splitkv_workspace_bytes.argtypes = [i, i, i, i, i]
        L.fa_splitkv_workspace_bytes.restype = sz
        L.fa_splitkv_default_splits.argtypes = [i, i, i, i, i, i]
        L.fa_splitkv_default_splits.restype = i
        L.fa_fwd_splitkv.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, i, vp, sz, vp]
        L.fa_fwd_splitkv.restype = i
        L.fa_fwd_splitkv_static.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, i, vp]
        L.fa_fwd_splitkv_static.restype = i
        L.fa_merge_partials.argtypes = [vp, vp, i, i, i, i, i, i, vp, vp, vp]
        L.fa_merge_partials.restype = i
        L.fa_fwd_gqa.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp, i, vp, sz, vp]
        L.fa_fwd_gqa.restype = i
        L.fa_fwd_mxfp8.argtypes = [vp] * 8 + [i, i, i, i, i, i, f, i, vp, ctypes.c_size_t, vp]
        L.fa_fwd_mxfp8.restype = i
        L.fa_bwd_workspace_bytes.argtypes = [i, i, i]
        L.fa_bwd_workspace_bytes.restype = sz
        L.fa_bwd.argtypes = [vp] * 9 + [i, i, i, i, i, i, f, i, vp, sz, vp]
        L.fa_bwd.restype = i
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().fa_status_string(int(status)).decode()


def _ptr(t) -> int:
    return 0 if t is None else t.data_ptr()


def _device(*tensors) -> torch.device:
    """The one device every given tensor (None entries skipped) lives on."""
    dev = None
    for t in tensors:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("every tensor must be a device tensor")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"tensors on different devices ({dev} and {t.device})")
    return dev


def _call(name: str, dev: torch.device, *args) -> int:
    """Enqueue a library entry point on `dev`: that device current, on its
    current torch stream (the last argument of every enqueuing entry point)."""
    with torch.cuda.device(dev):
        return getattr(lib(), name)(*args, torch.cuda.current_stream(dev).cuda_stream)


def _check_workspace(ws) -> int:
    """Size in bytes of a caller's workspace (0 for None); it must be a
    contiguous uint8 device tensor, so that numel() is its size in bytes."""
    if ws is None:
        return 0
    if ws.dtype != torch.uint8 or not ws.is_cuda or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 device tensor")
    return ws.numel()


def _check_out(t, dtype, shape, name):
    """A caller-provided output must be a contiguous device tensor of exactly
    this dtype and shape: the kernels write all of it and nothing else."""
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"{name} must be a contiguous {dtype} {tuple(shape)} device tensor")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return DTYPE_F32
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return DTYPE_FP8_E4M3
    raise TypeError(f"unsupported input dtype {t.dtype}")


def _check_qkv(q, k, v):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [B, H, N, d] tensor")
    if k.shape != v.shape or q.shape[0] != k.shape[0] or q.shape[2:] != k.shape[2:]:
        raise ValueError("q must be [B, Hq, N, d] and k, v [B, Hkv, N, d]")
    if k.shape[1] < 1 or q.shape[1] % k.shape[1] != 0:
        raise ValueError("the query heads must be a multiple of the key/value heads")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k and v must share a dtype")


def splitkv_chunk_keys(N: int, num_splits: int) -> int:
    """Keys per chunk of the split-KV forward (0 for invalid arguments)."""
    return int(lib().fa_splitkv_chunk_keys(int(N), int(num_splits)))


def splitkv_workspace_bytes(B: int, H: int, N: int, d: int, num_splits: int) -> int:
    """Device workspace bytes fa_fwd_splitkv needs (0 for invalid arguments)."""
    return int(lib().fa_splitkv_workspace_bytes(int(B), int(H), int(N), int(d), int(num_splits)))


def default_splits(B: int, H: int, N: int, d: int, causal: bool, dtype_code: int, device=None) -> int:
    """The number of key chunks the library picks for this shape on `device`
    (default: the current device)."""
    with torch.cuda.device(device if device is not None else torch.cuda.current_device()):
        return int(lib().fa_splitkv_default_splits(int(B), int(H), int(N), int(d),
                                                   1 if causal else 0, int(dtype_code)))


def fwd(q, k, v, causal: bool = False, scale: float | None = None, descales=None,
        out=None, lse=None, num_splits: int | None = None, workspace=None):
    """FlashAttention-2 forward. q: contiguous [B, Hq, N, d], k and v:
    contiguous [B, Hkv, N, d] device tensors (Hq a multiple of Hkv: grouped-
    query attention when Hkv < Hq), all float32, all bfloat16, or all FP8
    codes (uint8 or float8_e4m3fn) with descales of B*Hq + 2*B*Hkv float32
    values (q, k, v; [3, B*H] when Hkv == Hq). Returns (o, lse):
    o [B, Hq, N, d] (float32 for float32 inputs, bfloat16 otherwise) and
    lse [B, Hq, N] float32.

    num_splits: None lets the library choose (fa_splitkv_default_splits);
    1 runs the unsplit kernels (fa_fwd, or fa_fwd_gqa for Hkv < Hq); more runs
    the split-KV path with that many key chunks, in `workspace` (a uint8 device
    tensor of at least splitkv_workspace_bytes bytes) or in one allocated
    here."""
    _check_qkv(q, k, v)
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    code = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    odt = torch.float32 if code == DTYPE_F32 else torch.bfloat16
    if out is None:
        out = torch.empty((B, H, N, d), dtype=odt, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if out.dtype != odt or out.shape != q.shape or not out.is_contiguous():
        raise ValueError("out has the wrong dtype, shape or layout")
    if lse.dtype != torch.float32 or lse.shape != (B, H, N) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor")
    if code == DTYPE_FP8_E4M3:
        if descales is None:
            raise ValueError("FP8 inputs need descales (q, k, v per head)")
        if descales.dtype != torch.float32 or descales.numel() != B * H + 2 * B * Hkv \
                or not descales.is_contiguous() or not descales.is_cuda:
            raise ValueError("descales must be a contiguous float32 device tensor of "
                             "B*Hq + 2*B*Hkv values")
    ds = _ptr(descales) if code == DTYPE_FP8_E4M3 else None
    if num_splits is None:
        num_splits = default_splits(B, H, N, d, causal, code, q.device)
    if Hkv != H:
        need = splitkv_workspace_bytes(B, H, N, d, num_splits) if num_splits > 1 else 0
        if num_splits > 1 and workspace is None:
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
        ws_bytes = _check_workspace(workspace)
        dev = _device(q, k, v, out, lse, descales, workspace)
        st = _call("fa_fwd_gqa", dev, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Hkv, N, d,
                   1 if causal else 0, float(scale), code, ds, int(num_splits), _ptr(workspace), ws_bytes)
        if st != FA_OK:
            raise FAError(st, "fa_fwd_gqa")
        return out, lse
    if num_splits == 1 and workspace is None:
        dev = _device(q, k, v, out, lse, descales)
        st = _call("fa_fwd", dev, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, d,
                   1 if causal else 0, float(scale), code, ds)
        if st != FA_OK:
            raise FAError(st, "fa_fwd")
        return out, lse
    need = splitkv_workspace_bytes(B, H, N, d, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    ws_bytes = _check_workspace(workspace)
    dev = _device(q, k, v, out, lse, descales, workspace)
    st = _call("fa_fwd_splitkv", dev, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, d,
               1 if causal else 0, float(scale), code, ds, int(num_splits), _ptr(workspace), ws_bytes)
    if st != FA_OK:
        raise FAError(st, "fa_fwd_splitkv")
    return out, lse


def fwd_splitkv_static(q, k, v, num_splits: int, causal: bool = False, scale: float | None = None,
                       descales=None, out=None, lse=None):
    """The split-KV forward with its partials in the library's own static
    device scratch (fa_fwd_splitkv_static): no workspace, and the C call
    allocates nothing. q, k, v: contiguous [B, H, N, d] device tensors (no
    grouped-query form), dtypes and descales as fwd; out and lse may be given
    so that nothing is allocated here either. Raises FAError (FA_ERR_SCRATCH)
    when the partials exceed STATIC_SCRATCH_BYTES."""
    _check_qkv(q, k, v)
    B, H, N, d = q.shape
    if k.shape[1] != H:
        raise ValueError("fwd_splitkv_static takes as many key/value heads as query heads")
    code = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    odt = torch.float32 if code == DTYPE_F32 else torch.bfloat16
    if out is None:
        out = torch.empty((B, H, N, d), dtype=odt, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check_out(out, odt, (B, H, N, d), "out")
    _check_out(lse, torch.float32, (B, H, N), "lse")
    ds = None
    if code == DTYPE_FP8_E4M3:
        if descales is None:
            raise ValueError("FP8 inputs need descales (q, k, v per head)")
        if descales.dtype != torch.float32 or descales.numel() != 3 * B * H \
                or not descales.is_contiguous() or not descales.is_cuda:
            raise ValueError("descales must be a contiguous float32 device tensor of 3*B*H values")
        ds = _ptr(descales)
    dev = _device(q, k, v, out, lse, descales)
    st = _call("fa_fwd_splitkv_static", dev, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, d,
               1 if causal else 0, float(scale), code, ds, int(num_splits))
    if st != FA_OK:
        raise FAError(st, "fa_fwd_splitkv_static")
    return out, lse


def splitkv_partials(workspace, num_splits: int, B: int, H: int, N: int, d: int):
    """Views of the partial results fa_fwd_splitkv leaves in its workspace:
    (o_parts float32 [num_splits, B*H, N, d], lse_parts float32 [num_splits, B*H, N])."""
    n_o = num_splits * B * H * N * d
    f = workspace.view(torch.float32)
    return (f[:n_o].view(num_splits, B * H, N, d),
            f[n_o:n_o + num_splits * B * H * N].view(num_splits, B * H, N))


def merge_partials(o_parts, lse_parts, out_dtype=torch.bfloat16, out=None, lse=None):
    """Merge partial attention results over disjoint key sets.
    o_parts float32 [S, B*H, N, d], lse_parts float32 [S, B*H, N] (contiguous,
    on the device). Returns (o [B*H, N, d] of out_dtype float32 or bfloat16,
    lse float32 [B*H, N])."""
    if o_parts.dim() != 4 or lse_parts.dim() != 3:
        raise ValueError("o_parts must be [S, B*H, N, d] and lse_parts [S, B*H, N]")
    S, BH, N, d = o_parts.shape
    for name, t in (("o_parts", o_parts), ("lse_parts", lse_parts)):
        if t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 device tensor")
    if tuple(lse_parts.shape) != (S, BH, N):
        raise ValueError("lse_parts shape does not match o_parts")
    code = {torch.float32: DTYPE_F32, torch.bfloat16: DTYPE_BF16}.get(out_dtype)
    if code is None:
        raise TypeError("out_dtype must be float32 or bfloat16")
    if out is None:
        out = torch.empty((BH, N, d), dtype=out_dtype, device=o_parts.device)
    if lse is None:
        lse = torch.empty((BH, N), dtype=torch.float32, device=o_parts.device)
    _check_out(out, out_dtype, (BH, N, d), "out")
    _check_out(lse, torch.float32, (BH, N), "lse")
    dev = _device(o_parts, lse_parts, out, lse)
    st = _call("fa_merge_partials", dev, _ptr(o_parts), _ptr(lse_parts), S, 1, BH, N, d, code, _ptr(out),
               _ptr(lse))
    if st != FA_OK:
        raise FAError(st, "fa_merge_partials")
    return out, lse


def quantize_fp8(x, out=None, descale=None):
    """Per-head e4m3 quantisation of a contiguous [B, H, N, d] float32 or
    bfloat16 device tensor. Returns (codes uint8 [B, H, N, d],
    descale float32 [B*H])."""
    if not x.is_cuda or x.dim() != 4 or not x.is_contiguous():
        raise ValueError("x must be a contiguous [B, H, N, d] device tensor")
    B, H, N, d = x.shape
    if x.dtype == torch.bfloat16:
        code = DTYPE_BF16
    elif x.dtype == torch.float32:
        code = DTYPE_F32
    else:
        raise TypeError("quantize_fp8 takes float32 or bfloat16")
    if out is None:
        out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if descale is None:
        descale = torch.empty(B * H, dtype=torch.float32, device=x.device)
    _check_out(out, torch.uint8, x.shape, "out")
    _check_out(descale, torch.float32, (B * H,), "descale")
    dev = _device(x, out, descale)
    st = _call("fa_quantize_fp8", dev, _ptr(x), code, _ptr(out), _ptr(descale), B, H, N, d)
    if st != FA_OK:
        raise FAError(st, "fa_quantize_fp8")
    return out, descale


def quantize_fp8_rotated(x, signs, fold_inverse_d: bool, out=None, descale=None):
    """Randomised Hadamard rotation y = (x * signs) H of a contiguous
    [B, H, N, d] bfloat16 device tensor, then per-head e4m3 quantisation of y.
    signs: int8 [d] device tensor of +1 / -1. With fold_inverse_d the descale
    also carries 1/d (for Q). Returns (codes uint8 [B, H, N, d],
    descale float32 [B*H])."""
    if not x.is_cuda or x.dim() != 4 or not x.is_contiguous():
        raise ValueError("x must be a contiguous [B, H, N, d] device tensor")
    if x.dtype != torch.bfloat16:
        raise TypeError("quantize_fp8_rotated takes bfloat16")
    B, H, N, d = x.shape
    if (not signs.is_cuda or signs.dtype != torch.int8 or signs.dim() != 1
            or signs.numel() != d or not signs.is_contiguous()):
        raise ValueError("signs must be a contiguous int8 [d] device tensor")
    if out is None:
        out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if descale is None:
        descale = torch.empty(B * H, dtype=torch.float32, device=x.device)
    _check_out(out, torch.uint8, x.shape, "out")
    _check_out(descale, torch.float32, (B * H,), "descale")
    dev = _device(x, signs, out, descale)
    st = _call("fa_quantize_fp8_rotated", dev, _ptr(x), DTYPE_BF16, _ptr(signs), _ptr(out), _ptr(descale), B,
               H, N, d, 1 if fold_inverse_d else 0)
    if st != FA_OK:
        raise FAError(st, "fa_quantize_fp8_rotated")
    return out, descale


def quantize_qkv_fp8(q, k, v, signs=None):
    """Quantise Q, K and V per head. Returns (q8, k8, v8, descales): descales
    [3, B*H] when Q, K and V have the same heads, else the flat
    B*Hq + 2*B*Hkv layout fwd() takes for grouped-query attention.
    With signs (int8 [d] device tensor of +1 / -1), Q and K are rotated by
    the randomised Hadamard transform before quantising, 1/d folded into Q's
    descales; V is quantised as it is. fwd() on the result computes the same
    attention (the rotations cancel in Q K^T)."""
    B, H = q.shape[:2]
    Hkv = k.shape[1]
    flat = torch.empty(B * H + 2 * B * Hkv, dtype=torch.float32, device=q.device)
    if signs is None:
        q8, _ = quantize_fp8(q, descale=flat[:B * H])
        k8, _ = quantize_fp8(k, descale=flat[B * H:B * H + B * Hkv])
    else:
        q8, _ = quantize_fp8_rotated(q, signs, True, descale=flat[:B * H])
        k8, _ = quantize_fp8_rotated(k, signs, False, descale=flat[B * H:B * H + B * Hkv])
    v8, _ = quantize_fp8(v, descale=flat[B * H + B * Hkv:])
    return q8, k8, v8, (flat.view(3, B * H) if Hkv == H else flat)


def _float_code(x, name):
    if not x.is_cuda or x.dim() != 4 or not x.is_contiguous():
        raise ValueError(f"{name} must be a contiguous [B, H, N, d] device tensor")
    if x.dtype == torch.bfloat16:
        return DTYPE_BF16
    if x.dtype == torch.float32:
        return DTYPE_F32
    raise TypeError(f"{name} takes float32 or bfloat16")


def quantize_mxfp8_rows(x, signs=None, fold_inverse_d: bool = False, out=None, scales=None):
    """Per-block e4m3 quantisation of [B, H, N, d] rows in blocks of 32 head
    dims (for Q and K), optionally after the randomised Hadamard rotation
    (signs: int8 [d] device tensor; bfloat16 input) and a factor 1/d.
    Returns (codes uint8 [B, H, N, d], E8M0 scales uint8 [B, H, N, d/32])."""
    code = _float_code(x, "x")
    B, H, N, d = x.shape
    if signs is not None and (not signs.is_cuda or signs.dtype != torch.int8 or signs.dim() != 1
                              or signs.numel() != d or not signs.is_contiguous()):
        raise ValueError("signs must be a contiguous int8 [d] device tensor")
    if out is None:
        out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((B, H, N, max(d // 32, 1)), dtype=torch.uint8, device=x.device)
    _check_out(out, torch.uint8, x.shape, "out")
    _check_out(scales, torch.uint8, (B, H, N, max(d // 32, 1)), "scales")
    dev = _device(x, signs, out, scales)
    st = _call("fa_quantize_mxfp8_rows", dev, _ptr(x), code, _ptr(signs), 1 if fold_inverse_d else 0,
               _ptr(out), _ptr(scales), B, H, N, d)
    if st != FA_OK:
        raise FAError(st, "fa_quantize_mxfp8_rows")
    return out, scales


def quantize_mxfp8_keys(x, out=None, scales=None):
    """Per-block e4m3 quantisation of [B, H, N, d] in blocks of 32 keys of
    one column (for V). Returns (codes uint8 [B, H, N, d], E8M0 scales uint8
    [B, H, ceil(N/32), d])."""
    code = _float_code(x, "x")
    B, H, N, d = x.shape
    if out is None:
        out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((B, H, (N + 31) // 32, d), dtype=torch.uint8, device=x.device)
    _check_out(out, torch.uint8, x.shape, "out")
    _check_out(scales, torch.uint8, (B, H, (N + 31) // 32, d), "scales")
    dev = _device(x, out, scales)
    st = _call("fa_quantize_mxfp8_keys", dev, _ptr(x), code, _ptr(out), _ptr(scales), B, H, N, d)
    if st != FA_OK:
        raise FAError(st, "fa_quantize_mxfp8_keys")
    return out, scales


def quantize_qkv_mxfp8(q, k, v, signs=None):
    """Per-block quantisation of Q and K (row blocks) and V (key blocks).
    With signs, Q and K are rotated first and 1/d goes into Q's values, so
    fwd_mxfp8 on the result computes the same attention. Returns
    (q8, k8, v8, (q_scales, k_scales, v_scales))."""
    q8, qs = quantize_mxfp8_rows(q, signs=signs, fold_inverse_d=signs is not None)
    k8, ks = quantize_mxfp8_rows(k, signs=signs)
    v8, vs = quantize_mxfp8_keys(v)
    return q8, k8, v8, (qs, ks, vs)


def fwd_mxfp8(q, k, v, scales, causal: bool = False, scale: float | None = None, num_splits=None,
              workspace=None, out=None, lse=None):
    """FP8 forward on per-block codes (head dim 128). q: uint8 [B, Hq, N, d];
    k, v: [B, Hkv, N, d]; scales: (q_scales [B, Hq, N, d/32], k_scales
    [B, Hkv, N, d/32], v_scales [B, Hkv, ceil(N/32), d]) as the quantisers
    return them. Returns (o bf16 [B, Hq, N, d], lse float32 [B, Hq, N])."""
    _check_qkv(q, k, v)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    qs, ks, vs = scales
    for name, t, shape in (("q_scales", qs, (B, Hq, N, d // 32)), ("k_scales", ks, (B, Hkv, N, d // 32)),
                           ("v_scales", vs, (B, Hkv, (N + 31) // 32, d))):
        if not t.is_cuda or t.dtype != torch.uint8 or tuple(t.shape) != shape or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous uint8 {shape} device tensor")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if num_splits is None:
        num_splits = default_splits(B, Hq, N, d, causal, DTYPE_FP8_E4M3, q.device)
    o = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device) if out is None else out
    if lse is None:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    if (o.shape != q.shape or o.dtype != torch.bfloat16 or not o.is_contiguous()
            or tuple(lse.shape) != (B, Hq, N) or lse.dtype != torch.float32 or not lse.is_contiguous()):
        raise ValueError("out must be bf16 [B, Hq, N, d] and lse float32 [B, Hq, N], contiguous")
    if num_splits > 1 and workspace is None:
        need = splitkv_workspace_bytes(B, Hq, N, d, num_splits)
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    # the caller's workspace is passed with its own size: the library refuses
    # one that is too small
    ws_bytes = _check_workspace(workspace) if num_splits > 1 else 0
    dev = _device(q, k, v, qs, ks, vs, o, lse, workspace)
    st = _call("fa_fwd_mxfp8", dev, _ptr(q), _ptr(k), _ptr(v), _ptr(qs), _ptr(ks), _ptr(vs), _ptr(o),
               _ptr(lse), B, Hq, Hkv, N, d, 1 if causal else 0, float(scale), int(num_splits),
               _ptr(workspace) if num_splits > 1 else None, ws_bytes)
    if st != FA_OK:
        raise FAError(st, "fa_fwd_mxfp8")
    return o, lse


def bwd_workspace_bytes(B: int, H: int, N: int) -> int:
    """Device workspace bytes fa_bwd needs on the current device: 8 per query
    row, plus the fp32 partial dQ of its key chunks on grids too small to fill
    the device."""
    return int(lib().fa_bwd_workspace_bytes(int(B), int(H), int(N)))


def bwd(q, k, v, o, lse, do, causal: bool = False, scale: float | None = None,
        dq=None, dk=None, dv=None, workspace=None):
    """FlashAttention-2 backward (bf16). q, o, do: contiguous [B, Hq, N, d];
    k, v: [B, Hkv, N, d]; lse: float32 [B, Hq, N] from fwd. Returns
    (dq, dk, dv) in bfloat16 with the shapes of q, k, v."""
    _check_qkv(q, k, v)
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    if q.dtype != torch.bfloat16:
        raise TypeError("the backward takes bfloat16 tensors")
    for name, t in (("o", o), ("do", do)):
        if t.dtype != torch.bfloat16 or t.shape != q.shape or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{name} must be a contiguous bfloat16 device tensor shaped like q")
    if lse.dtype != torch.float32 or lse.shape != (B, H, N) or not lse.is_contiguous() or not lse.is_cuda:
        raise ValueError("lse must be a contiguous float32 [B, H, N] device tensor")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _check_out(t, torch.bfloat16, ref.shape, name)
    if workspace is None:
        workspace = torch.empty(max(bwd_workspace_bytes(B, H, N), 16), dtype=torch.uint8, device=q.device)
    ws_bytes = _check_workspace(workspace)
    dev = _device(q, k, v, o, do, lse, dq, dk, dv, workspace)
    st = _call("fa_bwd", dev, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk),
               _ptr(dv), B, H, Hkv, N, d, 1 if causal else 0, float(scale), DTYPE_BF16, _ptr(workspace),
               ws_bytes)
    if st != FA_OK:
        raise FAError(st, "fa_bwd")
    return dq, dk, dv
