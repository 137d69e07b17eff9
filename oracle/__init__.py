"""fp64 CPU oracle for exact attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The HIP library and its Python binding
never import it, and they share no code with it.

``liboracle.so`` is built from ``oracle.c`` (plain C, fp64, OpenMP). It computes
the textbook definition of attention, materialising S and P for every query row.
The FlashAttention pages say the tiled online algorithm reproduces that
definition exactly (mlapandio "FlashAttention: IO-aware exact attention",
Definition and "Four ideas"). ``online.py`` is a separate fp64 model of the
tiled recurrence in the pages' notation; the tests pin it to the definition.

Every array here is numpy float64, contiguous [B, H, N, d]; LSE and D are
[B, Hq, N].
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .build import LIB_PATH, build

_f64p = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(_f64p)


def _c64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


class Oracle:
    """ctypes front end of one build of the oracle library.

    ``lib_path`` defaults to the in-tree ``liboracle.so``; tests pass other builds
    (for example deliberately broken ones) to check that the pins catch them."""

    def __init__(self, lib_path: str | None = None):
        path = lib_path or LIB_PATH
        if lib_path is None and not os.path.exists(path):
            build()
        lib = ctypes.CDLL(path)
        lib.oracle_attn_fwd.restype = ctypes.c_int
        lib.oracle_attn_fwd.argtypes = [_f64p, _f64p, _f64p, _f64p, _f64p] + [ctypes.c_int] * 6 + [
            _i64p, ctypes.c_int, ctypes.c_int, ctypes.c_double]
        lib.oracle_attn_probs.restype = ctypes.c_int
        lib.oracle_attn_probs.argtypes = [_f64p, _f64p, _f64p] + [ctypes.c_int] * 6 + [
            _i64p, ctypes.c_int, ctypes.c_int, ctypes.c_double]
        lib.oracle_attn_bwd.restype = ctypes.c_int
        lib.oracle_attn_bwd.argtypes = [_f64p] * 10 + [ctypes.c_int] * 7 + [ctypes.c_double, ctypes.c_int]
        lib.oracle_attn_bwd_sampled.restype = ctypes.c_int
        lib.oracle_attn_bwd_sampled.argtypes = [_f64p] * 4 + [_i64p, ctypes.c_int, _i64p, ctypes.c_int] + [
            _f64p] * 3 + [ctypes.c_int] * 7 + [ctypes.c_double, ctypes.c_int]
        lib.oracle_round_bf16.restype = ctypes.c_int
        lib.oracle_round_bf16.argtypes = [_f64p, _f64p, ctypes.c_int64]
        lib.oracle_num_threads.restype = ctypes.c_int
        _u8p = ctypes.POINTER(ctypes.c_uint8)
        _f32p = ctypes.POINTER(ctypes.c_float)
        lib.oracle_e4m3_decode.restype = ctypes.c_int
        lib.oracle_e4m3_decode.argtypes = [_u8p, _f64p, ctypes.c_int64]
        lib.oracle_e4m3_encode.restype = ctypes.c_int
        lib.oracle_e4m3_encode.argtypes = [_f32p, _u8p, ctypes.c_int64]
        lib.oracle_quantize_e4m3_blocks.restype = ctypes.c_int
        lib.oracle_quantize_e4m3_blocks.argtypes = [_f32p, _u8p, _f32p, ctypes.c_int64] + [ctypes.c_int] * 3
        self._u8p, self._f32p = _u8p, _f32p
        self.lib = lib

    @staticmethod
    def _dims(q, k):
        B, Hq, Nq, d = q.shape
        Bk, Hkv, Nk, dk = k.shape
        if Bk != B or dk != d:
            raise ValueError("q and k disagree on batch or head dim")
        return B, Hq, Hkv, Nq, Nk, d

    def fwd(self, q, k, v, causal: bool, scale: float, qpos=None, window: int = 0):
        """O [B,Hq,Nq,d] and LSE [B,Hq,Nq]. ``qpos`` (int64 [Nq]) places query
        rows among the keys for the causal mask (default: row i is position i);
        ``window`` > 0 keeps only a causal row's `window` most recent positions."""
        q, k, v = _c64(q), _c64(k), _c64(v)
        B, Hq, Hkv, Nq, Nk, d = self._dims(q, k)
        o = np.empty_like(q)
        lse = np.empty((B, Hq, Nq), dtype=np.float64)
        qp = None
        if qpos is not None:
            qpos = np.ascontiguousarray(qpos, dtype=np.int64)
            if qpos.shape != (Nq,):
                raise ValueError("qpos must have one entry per query row")
            qp = qpos.ctypes.data_as(_i64p)
        rc = self.lib.oracle_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Nq,
                                      Nk, d, qp, int(bool(causal)), int(window), float(scale))
        if rc != 0:
            raise ValueError("oracle_attn_fwd rejected its arguments")
        return o, lse

    def probs(self, q, k, causal: bool, scale: float, qpos=None, window: int = 0):
        """Full probability matrix P [B,Hq,Nq,Nk] (small sizes only)."""
        q, k = _c64(q), _c64(k)
        B, Hq, Hkv, Nq, Nk, d = self._dims(q, k)
        p = np.empty((B, Hq, Nq, Nk), dtype=np.float64)
        qp = None
        if qpos is not None:
            qpos = np.ascontiguousarray(qpos, dtype=np.int64)
            qp = qpos.ctypes.data_as(_i64p)
        rc = self.lib.oracle_attn_probs(_ptr(q), _ptr(k), _ptr(p), B, Hq, Hkv, Nq, Nk, d, qp,
                                        int(bool(causal)), int(window), float(scale))
        if rc != 0:
            raise ValueError("oracle_attn_probs rejected its arguments")
        return p

    def bwd(self, q, k, v, do, causal: bool, scale: float, o_bf16: bool = False, window: int = 0):
        """Gradients of sum(do * O): returns dict dq, dk, dv, o, lse, D.

        ``o_bf16``: form D = rowsum(do * O) from O rounded to bfloat16, the
        format the forward stores O in; every other quantity stays exact.
        ``window``: sliding-window causal mask, as in ``fwd``."""
        q, k, v, do = _c64(q), _c64(k), _c64(v), _c64(do)
        B, Hq, Hkv, Nq, Nk, d = self._dims(q, k)
        if Nq != Nk:
            raise ValueError("backward needs queries and keys of one sequence")
        if do.shape != q.shape:
            raise ValueError("do must be shaped like q")
        dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
        o = np.empty_like(q)
        lse = np.empty((B, Hq, Nq), dtype=np.float64)
        D = np.empty_like(lse)
        rc = self.lib.oracle_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(dq), _ptr(dk),
                                      _ptr(dv), _ptr(o), _ptr(lse), _ptr(D), B, Hq, Hkv, Nq, d,
                                      int(bool(causal)), int(window), float(scale), int(bool(o_bf16)))
        if rc != 0:
            raise ValueError("oracle_attn_bwd rejected its arguments")
        return dict(dq=dq, dk=dk, dv=dv, o=o, lse=lse, D=D)

    def bwd_sampled(self, q, k, v, do, causal: bool, scale: float, rows, keys, o_bf16: bool = False,
                    window: int = 0):
        """dQ of the listed query rows [B,Hq,len(rows),d] and dK/dV of the listed
        keys [B,Hkv,len(keys),d]; every row still runs its full softmax."""
        q, k, v, do = _c64(q), _c64(k), _c64(v), _c64(do)
        B, Hq, Hkv, Nq, Nk, d = self._dims(q, k)
        if Nq != Nk or do.shape != q.shape:
            raise ValueError("backward needs one sequence and do shaped like q")
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        keys = np.ascontiguousarray(keys, dtype=np.int64)
        dq = np.empty((B, Hq, len(rows), d))
        dk = np.empty((B, Hkv, len(keys), d))
        dv = np.empty((B, Hkv, len(keys), d))
        rc = self.lib.oracle_attn_bwd_sampled(_ptr(q), _ptr(k), _ptr(v), _ptr(do), rows.ctypes.data_as(_i64p),
                                              len(rows), keys.ctypes.data_as(_i64p), len(keys), _ptr(dq),
                                              _ptr(dk), _ptr(dv), B, Hq, Hkv, Nq, d, int(bool(causal)),
                                              int(window), float(scale), int(bool(o_bf16)))
        if rc != 0:
            raise ValueError("oracle_attn_bwd_sampled rejected its arguments")
        return dict(dq=dq, dk=dk, dv=dv)

    def round_bf16(self, x):
        """Round float64 values to the nearest bfloat16 value (ties to even)."""
        x = _c64(x)
        y = np.empty_like(x)
        if self.lib.oracle_round_bf16(_ptr(x), _ptr(y), x.size) != 0:
            raise ValueError("oracle_round_bf16 rejected its arguments")
        return y

    # ---- 8-bit floating point with block scales (OCP E4M3; see oracle.c) ----

    def e4m3_decode(self, codes):
        """float64 values of E4M3 codes (uint8); the NaN codes give NaN."""
        c = np.ascontiguousarray(codes, dtype=np.uint8)
        y = np.empty(c.shape, dtype=np.float64)
        if self.lib.oracle_e4m3_decode(c.ctypes.data_as(self._u8p), _ptr(y), c.size) != 0:
            raise ValueError("oracle_e4m3_decode rejected its arguments")
        return y

    def e4m3_encode(self, x):
        """E4M3 codes of float32 values: nearest, ties to even, saturated at 448."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        c = np.empty(x.shape, dtype=np.uint8)
        if self.lib.oracle_e4m3_encode(x.ctypes.data_as(self._f32p), c.ctypes.data_as(self._u8p), x.size) != 0:
            raise ValueError("oracle_e4m3_encode rejected its arguments")
        return c

    def quantize_e4m3(self, x, rows: int):
        """Block-quantise a float32 [B, H, N, d] tensor, one scale per `rows`
        rows of each (b, h): returns (codes uint8 [B, H, N, d], scales float32
        [B, H, ceil(N / rows)]) with x ~ code * scale."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        B, H, N, d = x.shape
        nb = (N + rows - 1) // rows
        c = np.empty(x.shape, dtype=np.uint8)
        sc = np.empty((B, H, nb), dtype=np.float32)
        rc = self.lib.oracle_quantize_e4m3_blocks(x.ctypes.data_as(self._f32p), c.ctypes.data_as(self._u8p),
                                                  sc.ctypes.data_as(self._f32p), B * H, N, d, rows)
        if rc != 0:
            raise ValueError("oracle_quantize_e4m3_blocks rejected its arguments")
        return c, sc

    def dequantize_e4m3(self, codes, scales, rows: int):
        """Exact float64 values code * scale (a 4-bit by 24-bit significand
        product, exact in float64)."""
        v = self.e4m3_decode(codes)
        s = np.repeat(np.asarray(scales, dtype=np.float64), rows, axis=2)[:, :, :v.shape[2]]
        return v * s[..., None]

    def fwd_e4m3(self, q8, k8, v8, qs, ks, vs, rows: int, causal: bool, scale: float):
        """The attention definition on the dequantised block-scaled inputs."""
        return self.fwd(self.dequantize_e4m3(q8, qs, rows), self.dequantize_e4m3(k8, ks, rows),
                        self.dequantize_e4m3(v8, vs, rows), causal, scale)

    def num_threads(self) -> int:
        return int(self.lib.oracle_num_threads())


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def fwd(q, k, v, causal, scale, qpos=None, window=0):
    return default().fwd(q, k, v, causal, scale, qpos, window)


def bwd(q, k, v, do, causal, scale, o_bf16=False, window=0):
    return default().bwd(q, k, v, do, causal, scale, o_bf16, window)


def bwd_sampled(q, k, v, do, causal, scale, rows, keys, o_bf16=False, window=0):
    return default().bwd_sampled(q, k, v, do, causal, scale, rows, keys, o_bf16, window)


def probs(q, k, causal, scale, qpos=None, window=0):
    return default().probs(q, k, causal, scale, qpos, window)
