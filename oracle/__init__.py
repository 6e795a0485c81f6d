"""Python access to the float64 oracle (oracle.c).

TEST INFRASTRUCTURE: only tests/, the smoke check and the benchmark's
CPU-baseline leg import this package. The GPU library never does.

attention(): gathered softmax attention with per-head sinks, float64.
topk():      exact per-row top-k selection, ascending output, -1 padding.
Both follow the definitions written at the top of oracle.c.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

from . import build as _build

_F32, _BF16 = 0, 1
_lib = None


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load liboracle.so, compiling it first if it is missing or older than its source."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    lib_path = path or _build.LIB
    if path is None and (not os.path.exists(lib_path)
                         or os.path.getmtime(lib_path) < os.path.getmtime(_build.SRC)):
        _build.build()
    lib = ctypes.CDLL(lib_path)
    lib.oracle_attention.restype = ctypes.c_int
    lib.oracle_attention.argtypes = [
        ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int64, ctypes.c_void_p, ctypes.c_double, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int]
    lib.oracle_topk.restype = ctypes.c_int
    lib.oracle_topk.argtypes = [
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
        ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    if path is None:
        _lib = lib
    return lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def attention(dtype: str, q, k, v, idx, nsel, sinks, scale: float, shared_cache: bool,
              rows: Optional[range] = None, threads: int = 0, lib: Optional[ctypes.CDLL] = None):
    """Gathered softmax attention with sinks in float64.

    dtype "bf16": q, k, v are uint16 bfloat16 bit patterns; "f32": float32.
    q [R, H, D]; k, v [C, N, D] (C = R for per-row caches, C = 1 when shared);
    idx [R, kmax] int32; nsel [R] int32 or None; sinks [H] float32.
    Returns float64 [R, H, D]; with `rows` given, only those rows are computed
    and the others are left NaN.
    """
    lib = lib or load()
    code = {"f32": _F32, "bf16": _BF16}[dtype]
    et = np.float32 if code == _F32 else np.uint16
    q = np.ascontiguousarray(q, dtype=et)
    k = np.ascontiguousarray(k, dtype=et)
    v = np.ascontiguousarray(v, dtype=et)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    nsel_a = None if nsel is None else np.ascontiguousarray(nsel, dtype=np.int32)
    sinks = np.ascontiguousarray(sinks, dtype=np.float32)
    R, H, D = q.shape
    if k.shape != v.shape or k.shape[2] != D or idx.shape[0] != R or sinks.shape != (H,):
        raise ValueError("shape mismatch")
    if not shared_cache and k.shape[0] != R:
        raise ValueError("per-row caches need one cache per row")
    out = np.full((R, H, D), np.nan, dtype=np.float64)
    spans = [(0, R)] if rows is None else [(r, r + 1) for r in rows]
    for b, e in spans:
        rc = lib.oracle_attention(code, _ptr(q), _ptr(k), _ptr(v), k.shape[1], int(shared_cache),
                                  _ptr(idx), _ptr(nsel_a), idx.shape[1], _ptr(sinks), float(scale),
                                  R, H, D, _ptr(out), b, e, int(threads))
        if rc != 0:
            raise RuntimeError(f"oracle_attention failed with code {rc}")
    return out


def topk(scores, k: int, valid_len=None, lib: Optional[ctypes.CDLL] = None):
    """Exact top-k per row: returns (idx int32 [R, k] ascending with -1 tail, count int32 [R])."""
    lib = lib or load()
    scores = np.ascontiguousarray(scores, dtype=np.float32)
    R, n = scores.shape
    vl = None if valid_len is None else np.ascontiguousarray(valid_len, dtype=np.int32)
    idx = np.empty((R, k), dtype=np.int32)
    cnt = np.empty(R, dtype=np.int32)
    rc = lib.oracle_topk(_ptr(scores), R, n, n, _ptr(vl), int(k), _ptr(idx), _ptr(cnt))
    if rc != 0:
        raise RuntimeError(f"oracle_topk failed with code {rc}")
    return idx, cnt
