"""Exact scaled dot-product attention for AMD MI355X (gfx950).

Thin ctypes binding over the C-ABI library ``lib/libattn.so`` (see
``include/attn.h``). This module only marshals arguments: it checks tensor
shapes and types, allocates outputs with PyTorch (device memory is PyTorch's
job here) and passes raw device pointers and the current HIP stream to the
library. Every step of the computation runs in the library's HIP kernels;
there is no fallback path — if the library is missing, calls raise.
"""
from __future__ import annotations

import ctypes
import math
import os
import pathlib
from typing import Optional

__all__ = ["attn_fwd", "attn_fwd_fp8", "attn_bwd", "attn_bwd_noalloc", "attn_bwd_workspace_bytes", "attn_decode",
           "attn_decode_fp8kv",
           "attn_decode_workspace_bytes", "attn_status_string",
           "AttnError", "lib", "LIB_PATH", "DTYPE_F32", "DTYPE_BF16", "DTYPE_F16",
           "EXPORTED_SYMBOLS"]

LIB_PATH = pathlib.Path(__file__).resolve().parent / "lib" / "libattn.so"

ATTN_OK = 0
DTYPE_F32 = 0
DTYPE_BF16 = 1
DTYPE_F16 = 2
# Every function include/attn.h declares.
EXPORTED_SYMBOLS = ("attn_fwd", "attn_fwd_gqa", "attn_fwd_fp8", "attn_bwd", "attn_bwd_gqa", "attn_bwd_noalloc",
                    "attn_bwd_workspace_bytes", "attn_decode", "attn_decode_fp8kv",
                    "attn_decode_workspace_bytes", "attn_status_string", "attn_last_error")

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str = ""):
        self.status = status
        name = _status_name(status)
        super().__init__(f"{where} failed: {name}" + (f" ({detail})" if detail else ""))


def lib() -> ctypes.CDLL:
    """Load libattn.so (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not LIB_PATH.exists():
        raise RuntimeError(f"HIP attention library not found at {LIB_PATH}; "
                           "build it with exact_attention_24_amd.build.build()")
    L = ctypes.CDLL(str(LIB_PATH))
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, vp, vp]
    L.attn_fwd.restype = i32
    L.attn_fwd_gqa.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, i32, vp, vp]
    L.attn_fwd_gqa.restype = i32
    L.attn_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32,
                               i32, vp, vp]
    L.attn_fwd_fp8.restype = i32
    L.attn_bwd_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    L.attn_bwd_workspace_bytes.restype = sz
    L.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                           i32, i32, i32, i32, i32, f32, i32, vp, vp]
    L.attn_bwd.restype = i32
    L.attn_bwd_gqa.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                               i32, i32, i32, i32, i32, i32, f32, i32, vp, vp]
    L.attn_bwd_gqa.restype = i32
    L.attn_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                   i32, i32, i32, i32, i32, i32, f32, i32, vp, vp]
    L.attn_bwd_noalloc.restype = i32
    L.attn_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32]
    L.attn_decode_workspace_bytes.restype = sz
    L.attn_decode.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, i32, vp,
                              i32, vp, sz, vp]
    L.attn_decode.restype = i32
    L.attn_decode_fp8kv.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                    f32, i32, vp, i32, vp, sz, vp]
    L.attn_decode_fp8kv.restype = i32
    L.attn_status_string.argtypes = [i32]
    L.attn_status_string.restype = ctypes.c_char_p
    L.attn_last_error.argtypes = []
    L.attn_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def _status_name(status: int) -> str:
    try:
        return lib().attn_status_string(status).decode()
    except Exception:  # noqa: BLE001 - naming only
        return f"status {status}"


def attn_status_string(status: int) -> str:
    return lib().attn_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != ATTN_OK:
        detail = lib().attn_last_error().decode()
        raise AttnError(status, where, detail)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float16:
        return DTYPE_F16
    if t.dtype == torch.float32:
        return DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype}; expected bfloat16, float16 or float32")


def _stream_handle(device) -> int:
    import torch
    return torch.cuda.current_stream(device).cuda_stream


def _check_tensor(name: str, t, shape, dtype, device):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _seqlens_ptr(seqlens, B, device) -> int:
    import torch
    if seqlens is None:
        return 0
    _check_tensor("seqlens", seqlens, (B,), torch.int32, device)
    return seqlens.data_ptr()


def _kv_heads(q, k) -> int:
    """K/V head count: k is [B, H_kv, N, d] with H_kv dividing q's H."""
    if k is None or k.dim() != 4:
        raise ValueError("k must be a 4-d [B, H_kv, N, d] tensor")
    H, H_kv = q.shape[1], k.shape[1]
    if H_kv < 1 or H % H_kv != 0:
        raise ValueError(f"K/V head count {H_kv} must divide the query head count {H}")
    return H_kv


def attn_fwd(q, k, v, *, scale: Optional[float] = None, causal: bool = False,
             seqlens=None, out=None, lse=None, return_lse: bool = True):
    """O = softmax(scale * Q K^T) V over [B, H, N, d] device tensors.

    k and v may have fewer heads than q ([B, H_kv, N, d], H_kv dividing H):
    query head h then reads K/V head h // (H // H_kv) (grouped- or
    multi-query attention). Returns (O, LSE) with LSE fp32 [B, H, N] (natural
    log), or O alone when ``return_lse`` is False and no ``lse`` buffer is given.
    """
    import torch
    B, H, N, d = q.shape
    dev = q.device
    H_kv = _kv_heads(q, k)
    _check_tensor("q", q, (B, H, N, d), q.dtype, dev)
    for name, t in (("k", k), ("v", v)):
        _check_tensor(name, t, (B, H_kv, N, d), q.dtype, dev)
    code = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    _check_tensor("out", out, (B, H, N, d), q.dtype, dev)
    if lse is None and return_lse:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    if lse is not None:
        _check_tensor("lse", lse, (B, H, N), torch.float32, dev)
    lse_ptr = lse.data_ptr() if lse is not None else 0
    if H_kv == H:
        st = lib().attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse_ptr,
                            B, H, N, d, code, float(scale), int(bool(causal)),
                            _seqlens_ptr(seqlens, B, dev), _stream_handle(dev))
        _check(st, "attn_fwd")
    else:
        st = lib().attn_fwd_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse_ptr,
                                B, H, H_kv, N, d, code, float(scale), int(bool(causal)),
                                _seqlens_ptr(seqlens, B, dev), _stream_handle(dev))
        _check(st, "attn_fwd_gqa")
    return (out, lse) if lse is not None else out


def attn_fwd_fp8(q8, k8, v8, q_scale, k_scale, v_scale, *, scale: Optional[float] = None,
                 causal: bool = False, seqlens=None, out_dtype=None, out=None, lse=None):
    """Attention forward over FP8 E4M3 inputs on the FP8 matrix cores:
    Q = q8 * q_scale[..., None] (per token), K = k8 * k_scale, V = v8 * v_scale
    (per batch and K/V head). q8 is [B, H, N, 128], k8 and v8 [B, H_kv, N, 128]
    (torch.float8_e4m3fn or uint8, the same bytes); q_scale is fp32 [B, H, N],
    k_scale and v_scale fp32 [B, H_kv]. Returns (O, LSE) with O in out_dtype
    (torch.bfloat16 by default, or torch.float16) and LSE fp32 [B, H, N]."""
    import torch
    B, H, N, d = q8.shape
    dev = q8.device
    H_kv = _kv_heads(q8, k8)
    for name, t, shape in (("q8", q8, (B, H, N, d)), ("k8", k8, (B, H_kv, N, d)),
                           ("v8", v8, (B, H_kv, N, d))):
        if t.dtype not in (torch.uint8, getattr(torch, "float8_e4m3fn", torch.uint8)):
            raise TypeError(f"{name} must be float8_e4m3fn or uint8, not {t.dtype}")
        _check_tensor(name, t, shape, t.dtype, dev)
    _check_tensor("q_scale", q_scale, (B, H, N), torch.float32, dev)
    for name, t in (("k_scale", k_scale), ("v_scale", v_scale)):
        _check_tensor(name, t, (B, H_kv), torch.float32, dev)
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else torch.bfloat16
    if out_dtype not in (torch.bfloat16, torch.float16):
        raise TypeError(f"out_dtype must be torch.bfloat16 or torch.float16, not {out_dtype}")
    code = DTYPE_F16 if out_dtype == torch.float16 else DTYPE_BF16
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, H, N, d), dtype=out_dtype, device=dev)
    _check_tensor("out", out, (B, H, N, d), out_dtype, dev)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    _check_tensor("lse", lse, (B, H, N), torch.float32, dev)
    st = lib().attn_fwd_fp8(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), q_scale.data_ptr(),
                            k_scale.data_ptr(), v_scale.data_ptr(), out.data_ptr(), lse.data_ptr(),
                            B, H, H_kv, N, d, code, float(scale), int(bool(causal)),
                            _seqlens_ptr(seqlens, B, dev), _stream_handle(dev))
    _check(st, "attn_fwd_fp8")
    return out, lse


def attn_bwd_workspace_bytes(B: int, H: int, N: int, d: int, dtype_code: int = DTYPE_BF16) -> int:
    return int(lib().attn_bwd_workspace_bytes(B, H, N, d, dtype_code))


def attn_bwd(q, k, v, o, do, lse, *, scale: Optional[float] = None, causal: bool = False,
             seqlens=None, dq=None, dk=None, dv=None, workspace=None):
    """Recompute-based backward. Returns (dQ, dK, dV) in the input dtype; with
    grouped K/V heads dK, dV have k's shape and sum over each group."""
    import torch
    B, H, N, d = q.shape
    dev = q.device
    H_kv = _kv_heads(q, k)
    for name, t in (("q", q), ("o", o), ("do", do)):
        _check_tensor(name, t, (B, H, N, d), q.dtype, dev)
    for name, t in (("k", k), ("v", v)):
        _check_tensor(name, t, (B, H_kv, N, d), q.dtype, dev)
    _check_tensor("lse", lse, (B, H, N), torch.float32, dev)
    code = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _check_tensor("dq", dq, (B, H, N, d), q.dtype, dev)
    for name, t in (("dk", dk), ("dv", dv)):
        _check_tensor(name, t, (B, H_kv, N, d), q.dtype, dev)
    need = attn_bwd_workspace_bytes(B, H, N, d, code)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    if workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device buffer")
    nbytes = workspace.numel() * workspace.element_size()
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
            lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(), nbytes)
    tail = (code, float(scale), int(bool(causal)), _seqlens_ptr(seqlens, B, dev), _stream_handle(dev))
    if H_kv == H:
        st = lib().attn_bwd(*ptrs, B, H, N, d, *tail)
        _check(st, "attn_bwd")
    else:
        st = lib().attn_bwd_gqa(*ptrs, B, H, H_kv, N, d, *tail)
        _check(st, "attn_bwd_gqa")
    return dq, dk, dv


def attn_bwd_noalloc(q, k, v, o, do, lse, *, scale: Optional[float] = None, causal: bool = False,
                     seqlens=None, dq, dk, dv):
    """attn_bwd into caller-provided dq, dk, dv with no workspace: the library's
    static device scratch holds the backward's per-row statistics (at most
    2^21 = B*H*N query rows). Nothing is allocated, so it can run where
    allocation is not allowed (under graph capture, for instance). Calls that
    may overlap on one GPU share that scratch and must not run concurrently."""
    import torch
    B, H, N, d = q.shape
    dev = q.device
    H_kv = _kv_heads(q, k)
    for name, t in (("q", q), ("o", o), ("do", do), ("dq", dq)):
        _check_tensor(name, t, (B, H, N, d), q.dtype, dev)
    for name, t in (("k", k), ("v", v), ("dk", dk), ("dv", dv)):
        _check_tensor(name, t, (B, H_kv, N, d), q.dtype, dev)
    _check_tensor("lse", lse, (B, H, N), torch.float32, dev)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib().attn_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                                lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                B, H, H_kv, N, d, _dtype_code(q), float(scale), int(bool(causal)),
                                _seqlens_ptr(seqlens, B, dev), _stream_handle(dev))
    _check(st, "attn_bwd_noalloc")
    return dq, dk, dv


def attn_decode_workspace_bytes(B: int, H: int, H_kv: int, Nq: int, Nk: int, d: int,
                                dtype_code: int = DTYPE_BF16, num_splits: int = 0) -> int:
    return int(lib().attn_decode_workspace_bytes(B, H, H_kv, Nq, Nk, d, dtype_code, num_splits))


def attn_decode(q, k, v, *, scale: Optional[float] = None, causal: bool = False, kv_lens=None,
                num_splits: int = 0, out=None, lse=None, workspace=None):
    """Split-KV decode: q [B, H, Nq, d] (the last Nq positions of each sequence)
    against k, v [B, H_kv, Nk, d]. Returns (O [B, H, Nq, d], LSE [B, H, Nq])."""
    import torch
    B, H, Nq, d = q.shape
    dev = q.device
    H_kv = _kv_heads(q, k)
    Nk = k.shape[2]
    _check_tensor("q", q, (B, H, Nq, d), q.dtype, dev)
    for name, t in (("k", k), ("v", v)):
        _check_tensor(name, t, (B, H_kv, Nk, d), q.dtype, dev)
    code = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = torch.empty_like(q) if out is None else out
    _check_tensor("out", out, (B, H, Nq, d), q.dtype, dev)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=dev) if lse is None else lse
    _check_tensor("lse", lse, (B, H, Nq), torch.float32, dev)
    need = attn_decode_workspace_bytes(B, H, H_kv, Nq, Nk, d, code, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    if workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device buffer")
    nbytes = workspace.numel() * workspace.element_size()
    st = lib().attn_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                           B, H, H_kv, Nq, Nk, d, code, float(scale), int(bool(causal)),
                           _seqlens_ptr(kv_lens, B, dev), int(num_splits), workspace.data_ptr(),
                           nbytes, _stream_handle(dev))
    _check(st, "attn_decode")
    return out, lse


def attn_decode_fp8kv(q, k8, v8, k_scale, v_scale, *, scale: Optional[float] = None,
                      causal: bool = False, kv_lens=None, num_splits: int = 0, out=None, lse=None,
                      workspace=None):
    """Split-KV decode over an FP8 (E4M3) K/V cache with per-token fp32 scales:
    K = k8 * k_scale[..., None], V = v8 * v_scale[..., None]. k8, v8 are
    [B, H_kv, Nk, d] tensors of torch.float8_e4m3fn or uint8 (the same bytes);
    k_scale, v_scale are fp32 [B, H_kv, Nk]. Returns (O, LSE) like attn_decode."""
    import torch
    B, H, Nq, d = q.shape
    dev = q.device
    H_kv = _kv_heads(q, k8)
    Nk = k8.shape[2]
    _check_tensor("q", q, (B, H, Nq, d), q.dtype, dev)
    for name, t in (("k8", k8), ("v8", v8)):
        if t.dtype not in (torch.uint8, getattr(torch, "float8_e4m3fn", torch.uint8)):
            raise TypeError(f"{name} must be float8_e4m3fn or uint8, not {t.dtype}")
        _check_tensor(name, t, (B, H_kv, Nk, d), t.dtype, dev)
    for name, t in (("k_scale", k_scale), ("v_scale", v_scale)):
        _check_tensor(name, t, (B, H_kv, Nk), torch.float32, dev)
    code = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = torch.empty_like(q) if out is None else out
    _check_tensor("out", out, (B, H, Nq, d), q.dtype, dev)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=dev) if lse is None else lse
    _check_tensor("lse", lse, (B, H, Nq), torch.float32, dev)
    need = attn_decode_workspace_bytes(B, H, H_kv, Nq, Nk, d, code, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    if workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device buffer")
    nbytes = workspace.numel() * workspace.element_size()
    st = lib().attn_decode_fp8kv(q.data_ptr(), k8.data_ptr(), v8.data_ptr(), k_scale.data_ptr(),
                                 v_scale.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, H_kv, Nq,
                                 Nk, d, code, float(scale), int(bool(causal)),
                                 _seqlens_ptr(kv_lens, B, dev), int(num_splits), workspace.data_ptr(),
                                 nbytes, _stream_handle(dev))
    _check(st, "attn_decode_fp8kv")
    return out, lse
