"""TEST INFRASTRUCTURE ONLY: the fp64 CPU oracle for the exact attention forward.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never loads it and it
never loads the GPU library.

``attn_fwd`` / ``attn_fwd_online`` / ``attn_probs`` wrap ``liboracle.so``
(built from ``attn_oracle.c`` by :func:`build`); ``brute`` holds a pure-Python
brute force for tiny shapes.  Definitions and citations are in the C source.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "attn_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

_DT = {"fp16": 0, "bf16": 1}
_lib = None


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (plain -O2, no fast-math, OpenMP)."""
    if force or not os.path.exists(LIB):
        tmp = LIB + ".tmp"
        subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                        "-Wall", "-Werror", "-o", tmp, SRC, "-lm"], check=True)
        os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build(force=False)
        lib = ctypes.CDLL(LIB)
        i64, dbl, vp, ci = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p, ctypes.c_int
        lib.oracle_attn_fwd.argtypes = [vp, vp, vp, ci, i64, i64, i64, i64, dbl, ci,
                                        vp, i64, vp, vp]
        lib.oracle_attn_fwd.restype = ci
        lib.oracle_attn_fwd_qk.argtypes = [vp, vp, vp, ci, i64, i64, i64, i64, i64, dbl, ci,
                                           vp, i64, vp, vp]
        lib.oracle_attn_fwd_qk.restype = ci
        lib.oracle_attn_fwd_online.argtypes = [vp, vp, vp, ci, i64, i64, i64, i64, dbl,
                                               ci, i64, vp, vp]
        lib.oracle_attn_fwd_online.restype = ci
        lib.oracle_attn_probs.argtypes = [vp, vp, ci, i64, i64, i64, i64, dbl, ci, vp]
        lib.oracle_attn_probs.restype = ci
        lib.oracle_decode.argtypes = [vp, ci, i64, vp]
        lib.oracle_decode.restype = None
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = ci
        _lib = lib
    return _lib


def _words(a):
    a = np.ascontiguousarray(a, dtype=np.uint16)
    if a.ndim != 4:
        raise ValueError("expected [B,H,S,D] arrays of 16-bit words")
    return a


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def decode(bits, dtype: str) -> np.ndarray:
    """Exact float64 values of 16-bit words (the oracle's own decoder)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(b.shape, dtype=np.float64)
    _load().oracle_decode(b.ctypes.data, _DT[dtype], b.size, out.ctypes.data)
    return out


def attn_fwd(q, k, v, dtype: str, scale: float, causal: bool, rows=None):
    """Two-pass fp64 attention.

    q: uint16 [B,H,Sq,D]; k, v: uint16 [B,H,Skv,D] (Sq may differ from Skv;
    causal then keeps key j for query i iff j <= i + Skv - Sq).  rows: None
    (all rows; returns O [B,H,Sq,D], LSE [B,H,Sq]) or flat row indices
    (b*H + h)*Sq + i (returns O [n,D], LSE [n]).
    """
    q, k, v = _words(q), _words(k), _words(v)
    B, H, Sq, D = q.shape
    Skv = k.shape[2]
    if k.shape != (B, H, Skv, D) or v.shape != k.shape:
        raise ValueError("k and v must be [B,H,Skv,D] with q's B, H, D")
    if rows is None:
        o = np.empty((B, H, Sq, D), dtype=np.float64)
        lse = np.empty((B, H, Sq), dtype=np.float64)
        rp, n = None, 0
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        if rows.size and (rows.min() < 0 or rows.max() >= B * H * Sq):
            raise ValueError("row index out of range")
        o = np.empty((rows.size, D), dtype=np.float64)
        lse = np.empty((rows.size,), dtype=np.float64)
        rp, n = rows.ctypes.data, rows.size
    rc = _load().oracle_attn_fwd_qk(q.ctypes.data, k.ctypes.data, v.ctypes.data,
                                    _DT[dtype], B, H, Sq, Skv, D, float(scale),
                                    int(bool(causal)), rp, n, o.ctypes.data, lse.ctypes.data)
    if rc != 0:
        raise MemoryError("oracle scratch allocation failed")
    return o, lse


def attn_fwd_online(q, k, v, dtype: str, scale: float, causal: bool, block: int):
    """Blockwise online-softmax fp64 attention (all rows)."""
    q, k, v = _words(q), _words(k), _words(v)
    B, H, S, D = q.shape
    o = np.empty((B, H, S, D), dtype=np.float64)
    lse = np.empty((B, H, S), dtype=np.float64)
    rc = _load().oracle_attn_fwd_online(q.ctypes.data, k.ctypes.data, v.ctypes.data,
                                        _DT[dtype], B, H, S, D, float(scale),
                                        int(bool(causal)), int(block),
                                        o.ctypes.data, lse.ctypes.data)
    if rc != 0:
        raise ValueError("bad block size or allocation failure")
    return o, lse


def attn_probs(q, k, dtype: str, scale: float, causal: bool):
    """The fp64 softmax matrix P [B,H,S,S]."""
    q, k = _words(q), _words(k)
    B, H, S, D = q.shape
    p = np.empty((B, H, S, S), dtype=np.float64)
    rc = _load().oracle_attn_probs(q.ctypes.data, k.ctypes.data, _DT[dtype], B, H, S, D,
                                   float(scale), int(bool(causal)), p.ctypes.data)
    if rc != 0:
        raise MemoryError("oracle scratch allocation failed")
    return p
