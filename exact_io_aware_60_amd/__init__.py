"""Exact attention on AMD MI355X: Python binding of ``libflashattn.so``.

This module only marshals arguments. torch provides device memory and the
current stream; every step of the computation runs in the library's HIP
kernels. If the library is missing, ``lib()`` raises: there is no other
implementation to fall back to.

    o, lse = fwd(q, k, v, causal=True)                  # q [B,Hq,N,d], k/v [B,Hkv,N,d] bf16
    dq, dk, dv = bwd(q, k, v, o, lse, do, causal=True)
    o, lse = decode(q, k, v, causal=True)               # q [B,Hq,Nq,d], k/v [B,Hkv,Nk,d]

The entry points mirror ``include/flash_attn.h`` one to one.
"""
from __future__ import annotations

import ctypes
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libflashattn.so")

FA_OK, FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_HEADDIM, FA_ERR_ALIGN, FA_ERR_WORKSPACE, FA_ERR_HIP, FA_ERR_SCALE = (
    0, -1, -2, -3, -4, -5, -6, -7)
FA_ERR_SCRATCH = -8

EXPORTED = ("flash_attn_fwd", "flash_attn_bwd", "flash_attn_bwd_workspace_size", "flash_attn_strerror",
            "flash_attn_version", "flash_attn_bwd_preprocess", "flash_attn_bwd_dkdv", "flash_attn_bwd_dq",
            "flash_attn_decode", "flash_attn_decode_workspace_size", "flash_attn_fwd_varlen",
            "flash_attn_fwd_window", "flash_attn_bwd_window", "flash_attn_bwd_varlen",
            "flash_attn_quantize_e4m3", "flash_attn_decode_noalloc", "flash_attn_decode_noalloc_max_bytes",
            "flash_attn_quantize_e4m3_vt", "flash_attn_fwd_e4m3", "flash_attn_fwd_f32", "flash_attn_fwd_geometry")
BWD_STAGES = ("flash_attn_bwd_preprocess", "flash_attn_bwd_dq", "flash_attn_bwd_dkdv")

_lib = None
_vp = ctypes.c_void_p
_i = ctypes.c_int


class FlashAttnError(RuntimeError):
    def __init__(self, status: int, text: str):
        super().__init__(f"flash_attn status {status}: {text}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load the HIP library (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing; build it with exact_io_aware_60_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        L.flash_attn_fwd.restype = _i
        L.flash_attn_fwd.argtypes = [_vp] * 5 + [_i] * 6 + [ctypes.c_float, _vp]
        L.flash_attn_bwd_varlen.restype = _i
        L.flash_attn_bwd_varlen.argtypes = [_vp] * 10 + [_i] * 7 + [ctypes.c_float, _vp, ctypes.c_size_t, _vp]
        L.flash_attn_bwd_window.restype = _i
        L.flash_attn_bwd_window.argtypes = [_vp] * 9 + [_i] * 6 + [ctypes.c_float, _vp, ctypes.c_size_t, _vp]
        for name in ("flash_attn_bwd",) + BWD_STAGES:
            fn = getattr(L, name)
            fn.restype = _i
            fn.argtypes = [_vp] * 9 + [_i] * 6 + [ctypes.c_float, _vp, ctypes.c_size_t, _vp]
        L.flash_attn_bwd_workspace_size.restype = ctypes.c_size_t
        L.flash_attn_bwd_workspace_size.argtypes = [_i] * 6
        L.flash_attn_fwd_window.restype = _i
        L.flash_attn_fwd_window.argtypes = [_vp] * 5 + [_i] * 6 + [ctypes.c_float, _vp]
        L.flash_attn_fwd_varlen.restype = _i
        L.flash_attn_fwd_varlen.argtypes = [_vp] * 6 + [_i] * 7 + [ctypes.c_float, _vp]
        L.flash_attn_decode.restype = _i
        L.flash_attn_decode.argtypes = [_vp] * 6 + [_i] * 8 + [ctypes.c_float, _vp, ctypes.c_size_t, _vp]
        L.flash_attn_decode_noalloc.restype = _i
        L.flash_attn_decode_noalloc.argtypes = [_vp] * 6 + [_i] * 8 + [ctypes.c_float, _vp]
        L.flash_attn_decode_noalloc_max_bytes.restype = ctypes.c_size_t
        L.flash_attn_decode_noalloc_max_bytes.argtypes = []
        L.flash_attn_decode_workspace_size.restype = ctypes.c_size_t
        L.flash_attn_decode_workspace_size.argtypes = [_i] * 8
        L.flash_attn_quantize_e4m3.restype = _i
        L.flash_attn_quantize_e4m3.argtypes = [_vp] * 3 + [_i] * 4 + [_vp]
        L.flash_attn_quantize_e4m3_vt.restype = _i
        L.flash_attn_quantize_e4m3_vt.argtypes = [_vp] * 3 + [_i] * 4 + [_vp]
        L.flash_attn_fwd_e4m3.restype = _i
        L.flash_attn_fwd_e4m3.argtypes = [_vp] * 8 + [_i] * 6 + [ctypes.c_float, _i, _vp]
        L.flash_attn_fwd_f32.restype = _i
        L.flash_attn_fwd_f32.argtypes = [_vp] * 5 + [_i] * 6 + [ctypes.c_float, _vp]
        L.flash_attn_strerror.restype = ctypes.c_char_p
        L.flash_attn_strerror.argtypes = [_i]
        L.flash_attn_version.restype = ctypes.c_char_p
        L.flash_attn_version.argtypes = []
        L.flash_attn_fwd_geometry.restype = _i
        L.flash_attn_fwd_geometry.argtypes = [_i] * 6 + [_vp]
        _lib = L
    return _lib


def strerror(status: int) -> str:
    return lib().flash_attn_strerror(int(status)).decode()


def version() -> str:
    return lib().flash_attn_version().decode()


def fwd_geometry(B: int, Hq: int, Hkv: int, N: int, d: int, causal: bool = True) -> dict:
    """Launch shape of flash_attn_fwd for these arguments (host logic only)."""
    out = (ctypes.c_int * 5)()
    st = lib().flash_attn_fwd_geometry(B, Hq, Hkv, N, d, int(causal), out)
    if st != FA_OK:
        raise FlashAttnError(st, strerror(st))
    return dict(zip(("block_m", "block_n", "threads", "grid", "lds_bytes"), out))


def _check(status: int) -> None:
    if status != FA_OK:
        raise FlashAttnError(status, strerror(status))


# ------------------------------------------------------------------ raw C entry points
def fwd_raw(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, stream=None) -> int:
    """flash_attn_fwd on raw addresses (ints); returns the status code."""
    return lib().flash_attn_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, int(causal), float(scale), stream)


def bwd_raw(q, k, v, o, lse, do, dq, dk, dv, B, Hq, Hkv, N, d, causal, scale, workspace, workspace_bytes,
            stream=None) -> int:
    """flash_attn_bwd on raw addresses (ints); returns the status code."""
    return lib().flash_attn_bwd(q, k, v, o, lse, do, dq, dk, dv, B, Hq, Hkv, N, d, int(causal), float(scale),
                                workspace, workspace_bytes, stream)


def bwd_stage_raw(stage: int, q, k, v, o, lse, do, dq, dk, dv, B, Hq, Hkv, N, d, causal, scale, workspace,
                  workspace_bytes, stream=None) -> int:
    """One backward stage (0 = preprocess, 1 = dq, 2 = dkdv) on raw addresses; returns the status."""
    fn = getattr(lib(), BWD_STAGES[stage])
    return fn(q, k, v, o, lse, do, dq, dk, dv, B, Hq, Hkv, N, d, int(causal), float(scale), workspace,
              workspace_bytes, stream)


def bwd_varlen_raw(q, k, v, o, lse, do, dq, dk, dv, cu_seqlens, B, max_seqlen, total, Hq, Hkv, d, causal, scale,
                   workspace, workspace_bytes, stream=None) -> int:
    """flash_attn_bwd_varlen on raw addresses (ints); returns the status code."""
    return lib().flash_attn_bwd_varlen(q, k, v, o, lse, do, dq, dk, dv, cu_seqlens, B, max_seqlen, total, Hq, Hkv,
                                       d, int(causal), float(scale), workspace, workspace_bytes, stream)


def bwd_window_raw(q, k, v, o, lse, do, dq, dk, dv, B, Hq, Hkv, N, d, window, scale, workspace, workspace_bytes,
                   stream=None) -> int:
    """flash_attn_bwd_window on raw addresses (ints); returns the status code."""
    return lib().flash_attn_bwd_window(q, k, v, o, lse, do, dq, dk, dv, B, Hq, Hkv, N, d, int(window), float(scale),
                                       workspace, workspace_bytes, stream)


def bwd_workspace_size(B, Hq, Hkv, N, d, causal) -> int:
    return int(lib().flash_attn_bwd_workspace_size(B, Hq, Hkv, N, d, int(causal)))


def fwd_window_raw(q, k, v, o, lse, B, Hq, Hkv, N, d, window, scale, stream=None) -> int:
    """flash_attn_fwd_window on raw addresses (ints); returns the status code."""
    return lib().flash_attn_fwd_window(q, k, v, o, lse, B, Hq, Hkv, N, d, int(window), float(scale), stream)


def fwd_varlen_raw(q, k, v, o, lse, cu_seqlens, B, max_seqlen, total, Hq, Hkv, d, causal, scale,
                   stream=None) -> int:
    """flash_attn_fwd_varlen on raw addresses (ints); returns the status code."""
    return lib().flash_attn_fwd_varlen(q, k, v, o, lse, cu_seqlens, B, max_seqlen, total, Hq, Hkv, d, int(causal),
                                       float(scale), stream)


def decode_raw(q, k, v, o, lse, seqlens_k, B, Hq, Hkv, Nq, Nk, d, causal, scale, workspace, workspace_bytes,
               stream=None, window: int = 0) -> int:
    """flash_attn_decode on raw addresses (ints; seqlens_k may be None); returns the status code."""
    return lib().flash_attn_decode(q, k, v, o, lse, seqlens_k, B, Hq, Hkv, Nq, Nk, d, int(causal), int(window),
                                   float(scale), workspace, workspace_bytes, stream)


def decode_noalloc_raw(q, k, v, o, lse, seqlens_k, B, Hq, Hkv, Nq, Nk, d, causal, scale, stream=None,
                       window: int = 0) -> int:
    """flash_attn_decode_noalloc on raw addresses (ints; seqlens_k may be None); returns the status code."""
    return lib().flash_attn_decode_noalloc(q, k, v, o, lse, seqlens_k, B, Hq, Hkv, Nq, Nk, d, int(causal),
                                           int(window), float(scale), stream)


def decode_noalloc_max_bytes() -> int:
    return int(lib().flash_attn_decode_noalloc_max_bytes())


def quantize_e4m3_raw(x, codes, scales, BH, N, d, rows, stream=None) -> int:
    """flash_attn_quantize_e4m3 on raw addresses (ints); returns the status code."""
    return lib().flash_attn_quantize_e4m3(x, codes, scales, BH, N, d, rows, stream)


def quantize_e4m3_vt_raw(x, codes_t, scales, BH, N, d, rows, stream=None) -> int:
    """flash_attn_quantize_e4m3_vt on raw addresses (ints); returns the status code."""
    return lib().flash_attn_quantize_e4m3_vt(x, codes_t, scales, BH, N, d, rows, stream)


def fwd_e4m3_raw(q8, qs, k8, ks, v8t, vs, o, lse, B, Hq, Hkv, N, d, causal, scale, rows, stream=None) -> int:
    """flash_attn_fwd_e4m3 on raw addresses (ints); returns the status code."""
    return lib().flash_attn_fwd_e4m3(q8, qs, k8, ks, v8t, vs, o, lse, B, Hq, Hkv, N, d, int(causal), float(scale),
                                     int(rows), stream)


def fwd_f32_raw(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, stream=None) -> int:
    """flash_attn_fwd_f32 on raw addresses (ints); returns the status code."""
    return lib().flash_attn_fwd_f32(q, k, v, o, lse, B, Hq, Hkv, N, d, int(causal), float(scale), stream)


def decode_workspace_size(B, Hq, Hkv, Nq, Nk, d, causal, window: int = 0) -> int:
    return int(lib().flash_attn_decode_workspace_size(B, Hq, Hkv, Nq, Nk, d, int(causal), int(window)))


# ------------------------------------------------------------------ torch front end
def _dims(q, k):
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    B, Hq, N, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if (Bk, Nk, dk) != (B, N, d):
        raise ValueError("q and k/v must agree on B, N and d")
    return B, Hq, Hkv, N, d


def _checked(t, name):
    import torch
    if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous bfloat16 tensor on the GPU")
    return t


def _stream(t):
    import torch
    return torch.cuda.current_stream(t.device).cuda_stream


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


def fwd(q, k, v, causal: bool = True, scale: float | None = None, out=None, lse=None):
    """Forward pass. Returns (o bf16 [B,Hq,N,d], lse fp32 [B,Hq,N])."""
    import torch
    B, Hq, Hkv, N, d = _dims(q, k)
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _checked(t, name)
    if v.shape != k.shape:
        raise ValueError("v must be shaped like k")
    scale = default_scale(d) if scale is None else scale
    o = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _check(fwd_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, Hq, Hkv, N, d,
                   causal, scale, _stream(q)))
    return o, lse


def fwd_f32(q, k, v, causal: bool = True, scale: float | None = None, out=None, lse=None):
    """Forward pass on fp32 inputs. Returns (o fp32 [B,Hq,N,d], lse fp32 [B,Hq,N])."""
    import torch
    B, Hq, Hkv, N, d = _dims(q, k)
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        if t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 tensor on the GPU")
    if v.shape != k.shape:
        raise ValueError("v must be shaped like k")
    scale = default_scale(d) if scale is None else scale
    o = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _check(fwd_f32_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, Hq, Hkv, N, d,
                       causal, scale, _stream(q)))
    return o, lse


def fwd_window(q, k, v, window: int, scale: float | None = None, out=None, lse=None):
    """Forward pass with a sliding-window causal mask (row i sees keys i - window < j <= i).
    Returns (o bf16 [B,Hq,N,d], lse fp32 [B,Hq,N])."""
    import torch
    B, Hq, Hkv, N, d = _dims(q, k)
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _checked(t, name)
    if v.shape != k.shape:
        raise ValueError("v must be shaped like k")
    scale = default_scale(d) if scale is None else scale
    o = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _check(fwd_window_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, Hq, Hkv, N, d,
                          window, scale, _stream(q)))
    return o, lse


def bwd(q, k, v, o, lse, do, causal: bool = True, scale: float | None = None, workspace=None):
    """Backward pass for the loss sum(do * O). Returns (dq, dk, dv), bf16."""
    import torch
    B, Hq, Hkv, N, d = _dims(q, k)
    for t, name in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (do, "do")):
        _checked(t, name)
    if lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != (B, Hq, N):
        raise ValueError("lse must be contiguous float32 [B, Hq, N]")
    scale = default_scale(d) if scale is None else scale
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws_bytes = bwd_workspace_size(B, Hq, Hkv, N, d, causal)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=q.device)
    _check(bwd_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
                   dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, Hq, Hkv, N, d, causal, scale,
                   workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(q)))
    return dq, dk, dv


def decode(q, k, v, causal: bool = True, scale: float | None = None, workspace=None, out=None, lse=None,
           seqlens_k=None, window: int = 0):
    """Attention of the newest Nq query rows over a cache of Nk keys.

    q [B, Hq, Nq, d], k/v [B, Hkv, Nk, d] bf16. seqlens_k: optional int32
    device tensor [B], the cache rows in use per batch entry (default: all
    Nk). Causal: row i is token L_b - Nq + i; window > 0 keeps its `window`
    most recent keys. Returns (o bf16 [B,Hq,Nq,d], lse fp32 [B,Hq,Nq])."""
    import torch
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    B, Hq, Nq, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if (Bk, dk) != (B, d) or v.shape != k.shape:
        raise ValueError("q and k/v must agree on B and d, and v must be shaped like k")
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _checked(t, name)
    sl_ptr = None
    if seqlens_k is not None:
        if (seqlens_k.dtype != torch.int32 or not seqlens_k.is_cuda or not seqlens_k.is_contiguous()
                or tuple(seqlens_k.shape) != (B,)):
            raise ValueError("seqlens_k must be a contiguous int32 GPU tensor of shape [B]")
        sl_ptr = seqlens_k.data_ptr()
    scale = default_scale(d) if scale is None else scale
    o = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device) if lse is None else lse
    ws_bytes = decode_workspace_size(B, Hq, Hkv, Nq, Nk, d, causal, window)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(decode_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), sl_ptr, B, Hq, Hkv,
                      Nq, Nk, d, causal, scale, ws_ptr, ws_len, _stream(q), window))
    return o, lse


def decode_noalloc(q, k, v, out, lse, causal: bool = True, scale: float | None = None, seqlens_k=None,
                   window: int = 0):
    """decode() through flash_attn_decode_noalloc: the caller passes the outputs
    (o bf16 [B,Hq,Nq,d], lse fp32 [B,Hq,Nq]); the partial results go to the
    library's static per-GPU scratch, so nothing is allocated here or in the
    library. Overlapping calls on one GPU race (the scratch is shared)."""
    import torch
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    B, Hq, Nq, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if (Bk, dk) != (B, d) or v.shape != k.shape:
        raise ValueError("q and k/v must agree on B and d, and v must be shaped like k")
    for t, name in ((q, "q"), (k, "k"), (v, "v"), (out, "out")):
        _checked(t, name)
    if tuple(out.shape) != (B, Hq, Nq, d):
        raise ValueError("out must be shaped like q")
    if (lse.dtype != torch.float32 or not lse.is_cuda or not lse.is_contiguous()
            or tuple(lse.shape) != (B, Hq, Nq)):
        raise ValueError("lse must be a contiguous float32 GPU tensor of shape [B, Hq, Nq]")
    sl_ptr = None
    if seqlens_k is not None:
        if (seqlens_k.dtype != torch.int32 or not seqlens_k.is_cuda or not seqlens_k.is_contiguous()
                or tuple(seqlens_k.shape) != (B,)):
            raise ValueError("seqlens_k must be a contiguous int32 GPU tensor of shape [B]")
        sl_ptr = seqlens_k.data_ptr()
    scale = default_scale(d) if scale is None else scale
    _check(decode_noalloc_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), sl_ptr, B,
                              Hq, Hkv, Nq, Nk, d, causal, scale, _stream(q), window))
    return out, lse


def fwd_varlen(q, k, v, cu_seqlens, max_seqlen: int, causal: bool = True, scale: float | None = None, out=None,
               lse=None):
    """Forward pass over packed sequences: q [Hq, total, d], k/v [Hkv, total, d] bf16,
    cu_seqlens int32 [B + 1] on the GPU (sequence b is rows cu_seqlens[b] ..
    cu_seqlens[b+1]-1). Returns (o bf16 [Hq, total, d], lse fp32 [Hq, total])."""
    import torch
    if q.dim() != 3 or k.dim() != 3 or v.shape != k.shape:
        raise ValueError("q must be [Hq, total, d] and k, v [Hkv, total, d]")
    Hq, total, d = q.shape
    Hkv = k.shape[0]
    if k.shape[1:] != (total, d):
        raise ValueError("q and k/v must agree on total and d")
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _checked(t, name)
    if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_cuda or not cu_seqlens.is_contiguous() \
            or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be a contiguous int32 GPU tensor of shape [B + 1]")
    B = cu_seqlens.numel() - 1
    scale = default_scale(d) if scale is None else scale
    o = torch.empty_like(q) if out is None else out
    lse = torch.empty((Hq, total), dtype=torch.float32, device=q.device) if lse is None else lse
    _check(fwd_varlen_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                          cu_seqlens.data_ptr(), B, int(max_seqlen), total, Hq, Hkv, d, causal, scale, _stream(q)))
    return o, lse


def bwd_window(q, k, v, o, lse, do, window: int, scale: float | None = None, workspace=None):
    """Backward pass of fwd_window (same window). Returns (dq, dk, dv), bf16."""
    import torch
    B, Hq, Hkv, N, d = _dims(q, k)
    for t, name in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (do, "do")):
        _checked(t, name)
    if lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != (B, Hq, N):
        raise ValueError("lse must be contiguous float32 [B, Hq, N]")
    scale = default_scale(d) if scale is None else scale
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws_bytes = bwd_workspace_size(B, Hq, Hkv, N, d, True)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=q.device)
    _check(bwd_window_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
                          dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, Hq, Hkv, N, d, window, scale,
                          workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(q)))
    return dq, dk, dv


def bwd_varlen(q, k, v, o, lse, do, cu_seqlens, max_seqlen: int, causal: bool = True, scale: float | None = None,
               workspace=None):
    """Backward pass of fwd_varlen (causal or not): q/o/do [Hq, total, d], k/v [Hkv, total, d], lse [Hq, total].
    Returns (dq, dk, dv), bf16, in the same packed layout."""
    import torch
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("q must be [Hq, total, d] and k, v [Hkv, total, d]")
    Hq, total, d = q.shape
    Hkv = k.shape[0]
    for t, name in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (do, "do")):
        _checked(t, name)
    if lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != (Hq, total):
        raise ValueError("lse must be contiguous float32 [Hq, total]")
    if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_cuda or cu_seqlens.dim() != 1:
        raise ValueError("cu_seqlens must be an int32 GPU tensor of shape [B + 1]")
    scale = default_scale(d) if scale is None else scale
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws_bytes = bwd_workspace_size(1, Hq, Hkv, total, d, causal)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=q.device)
    _check(bwd_varlen_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
                          dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), cu_seqlens.data_ptr(), cu_seqlens.numel() - 1,
                          int(max_seqlen), total, Hq, Hkv, d, causal, scale, workspace.data_ptr(),
                          workspace.numel() * workspace.element_size(), _stream(q)))
    return dq, dk, dv


def quantize_e4m3(x, rows: int = 128):
    """Block-quantise a contiguous bf16 [..., N, d] GPU tensor to OCP E4M3 codes
    with one fp32 scale per run of `rows` rows of each leading slab (the last
    run ragged): returns (codes uint8 [..., N, d], scales float32
    [..., ceil(N / rows)]) with x ~ code * scale. See flash_attn_quantize_e4m3."""
    import torch
    _checked(x, "x")
    if x.dim() < 2:
        raise ValueError("x must be [..., N, d]")
    N, d = x.shape[-2], x.shape[-1]
    BH = x.numel() // max(N * d, 1)
    codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    rows = int(rows)
    nruns = -(-N // rows) if rows > 0 else 1          # rows < 1 is rejected by the library
    scales = torch.empty((*x.shape[:-2], nruns), dtype=torch.float32, device=x.device)
    _check(quantize_e4m3_raw(x.data_ptr(), codes.data_ptr(), scales.data_ptr(), BH, N, d, rows,
                             torch.cuda.current_stream().cuda_stream))
    return codes, scales


def quantize_e4m3_vt(v, rows: int = 128):
    """flash_attn_quantize_e4m3_vt: V's codes transposed for fwd_e4m3. v is a
    contiguous bf16 [..., N, d] GPU tensor; returns (codes_t uint8
    [..., d, Np], Np = N rounded up to 64, keys of every 64-key group in the
    forward's operand order; scales float32 [..., ceil(N / rows)])."""
    import torch
    _checked(v, "v")
    if v.dim() < 2:
        raise ValueError("v must be [..., N, d]")
    N, d = v.shape[-2], v.shape[-1]
    BH = v.numel() // max(N * d, 1)
    Np = -(-N // 64) * 64
    codes_t = torch.empty((*v.shape[:-2], d, Np), dtype=torch.uint8, device=v.device)
    rows = int(rows)
    nruns = -(-N // rows) if rows > 0 else 1
    scales = torch.empty((*v.shape[:-2], nruns), dtype=torch.float32, device=v.device)
    _check(quantize_e4m3_vt_raw(v.data_ptr(), codes_t.data_ptr(), scales.data_ptr(), BH, N, d, rows,
                                torch.cuda.current_stream().cuda_stream))
    return codes_t, scales


def fwd_e4m3(q8, q_scales, k8, k_scales, v8t, v_scales, rows: int, causal: bool = True, scale: float | None = None,
             out=None, lse=None):
    """Forward on 8-bit inputs (flash_attn_fwd_e4m3): q8 [B,Hq,N,d], k8
    [B,Hkv,N,d] uint8 E4M3 codes with fp32 run scales, v8t [B,Hkv,d,Np] from
    quantize_e4m3_vt. Returns (o bf16 [B,Hq,N,d], lse fp32 [B,Hq,N])."""
    import torch
    for t, name in ((q8, "q8"), (k8, "k8"), (v8t, "v8t")):
        if t.dtype != torch.uint8 or not t.is_cuda or not t.is_contiguous() or t.dim() != 4:
            raise ValueError(f"{name} must be a contiguous 4-d uint8 GPU tensor")
    for t, name in ((q_scales, "q_scales"), (k_scales, "k_scales"), (v_scales, "v_scales")):
        if t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 GPU tensor")
    B, Hq, N, d = q8.shape
    Hkv = k8.shape[1]
    Np = -(-N // 64) * 64
    if tuple(k8.shape) != (B, Hkv, N, d) or tuple(v8t.shape) != (B, Hkv, d, Np):
        raise ValueError("k8 must be [B, Hkv, N, d] and v8t [B, Hkv, d, Np]")
    nruns = -(-N // int(rows)) if rows > 0 else 1
    if (tuple(q_scales.shape) != (B, Hq, nruns) or tuple(k_scales.shape) != (B, Hkv, nruns)
            or tuple(v_scales.shape) != (B, Hkv, nruns)):
        raise ValueError("scale arrays must be [B, H, ceil(N / rows)]")
    scale = default_scale(d) if scale is None else scale
    o = torch.empty((B, Hq, N, d), dtype=torch.bfloat16, device=q8.device) if out is None else out
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q8.device) if lse is None else lse
    _check(fwd_e4m3_raw(q8.data_ptr(), q_scales.data_ptr(), k8.data_ptr(), k_scales.data_ptr(), v8t.data_ptr(),
                        v_scales.data_ptr(), o.data_ptr(), lse.data_ptr(), B, Hq, Hkv, N, d, causal, scale, rows,
                        _stream(q8)))
    return o, lse
