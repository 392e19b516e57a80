"""TEST INFRASTRUCTURE ONLY: the fp64 CPU oracle for the exact attention forward.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never loads it and it
never loads the GPU library.

``attn_fwd`` / ``attn_fwd_online`` / ``attn_probs`` / ``attn_bwd`` (and the
float64-input ``attn_fwd_f64`` / ``attn_bwd_f64``) wrap ``liboracle.so``
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
        lib.oracle_attn_fwd_f64.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, dbl, ci, vp, vp]
        lib.oracle_attn_fwd_f64.restype = ci
        lib.oracle_attn_bwd_f64.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, dbl, ci,
                                            vp, vp, vp, vp]
        lib.oracle_attn_bwd_f64.restype = ci
        lib.oracle_attn_bwd.argtypes = [vp, vp, vp, vp, ci, i64, i64, i64, i64, i64, dbl, ci,
                                        vp, vp, vp, vp]
        lib.oracle_attn_bwd.restype = ci
        lib.oracle_attn_bwd_rows.argtypes = [vp, vp, vp, vp, ci, i64, i64, i64, i64, i64, dbl, ci,
                                             vp, i64, vp, vp]
        lib.oracle_attn_bwd_rows.restype = ci
        lib.oracle_attn_bwd_keys.argtypes = [vp, vp, vp, vp, ci, i64, i64, i64, i64, i64, dbl, ci,
                                             vp, i64, vp, vp]
        lib.oracle_attn_bwd_keys.restype = ci
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


def _f64(a):
    a = np.ascontiguousarray(a, dtype=np.float64)
    if a.ndim != 4:
        raise ValueError("expected [B,H,S,D] float64 arrays")
    return a


def _qkv_shapes(q, k, v, *more):
    B, H, Sq, D = q.shape
    Skv = k.shape[2]
    if k.shape != (B, H, Skv, D) or v.shape != k.shape:
        raise ValueError("k and v must be [B,H,Skv,D] with q's B, H, D")
    for t in more:
        if t.shape != q.shape:
            raise ValueError("dO must have q's shape")
    return B, H, Sq, Skv, D


def attn_fwd_f64(q, k, v, scale: float, causal: bool):
    """The forward definition on float64 arrays: O [B,H,Sq,D], LSE [B,H,Sq]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, Sq, Skv, D = _qkv_shapes(q, k, v)
    o = np.empty((B, H, Sq, D), dtype=np.float64)
    lse = np.empty((B, H, Sq), dtype=np.float64)
    rc = _load().oracle_attn_fwd_f64(q.ctypes.data, k.ctypes.data, v.ctypes.data, B, H, Sq, Skv,
                                     D, float(scale), int(bool(causal)), o.ctypes.data,
                                     lse.ctypes.data)
    if rc != 0:
        raise MemoryError("oracle scratch allocation failed")
    return o, lse


def _bwd_out(B, H, Sq, Skv, D):
    return (np.empty((B, H, Sq, D)), np.empty((B, H, Skv, D)), np.empty((B, H, Skv, D)),
            np.empty((B, H, Sq)))


def attn_bwd_f64(q, k, v, do, scale: float, causal: bool):
    """The backward on float64 arrays: dQ, dK, dV and D_i = rowsum(dP * P)."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, H, Sq, Skv, D = _qkv_shapes(q, k, v, do)
    dq, dk, dv, delta = _bwd_out(B, H, Sq, Skv, D)
    rc = _load().oracle_attn_bwd_f64(q.ctypes.data, k.ctypes.data, v.ctypes.data, do.ctypes.data,
                                     B, H, Sq, Skv, D, float(scale), int(bool(causal)),
                                     dq.ctypes.data, dk.ctypes.data, dv.ctypes.data,
                                     delta.ctypes.data)
    if rc != 0:
        raise MemoryError("oracle scratch allocation failed")
    return dq, dk, dv, delta


def attn_bwd(q, k, v, do, dtype: str, scale: float, causal: bool):
    """The backward of 16-bit inputs q, k, v, dO (uint16 words of `dtype`),
    computed in float64: dQ [B,H,Sq,D], dK, dV [B,H,Skv,D], D_i [B,H,Sq]."""
    q, k, v, do = _words(q), _words(k), _words(v), _words(do)
    B, H, Sq, Skv, D = _qkv_shapes(q, k, v, do)
    dq, dk, dv, delta = _bwd_out(B, H, Sq, Skv, D)
    rc = _load().oracle_attn_bwd(q.ctypes.data, k.ctypes.data, v.ctypes.data, do.ctypes.data,
                                 _DT[dtype], B, H, Sq, Skv, D, float(scale), int(bool(causal)),
                                 dq.ctypes.data, dk.ctypes.data, dv.ctypes.data, delta.ctypes.data)
    if rc != 0:
        raise MemoryError("oracle scratch allocation failed")
    return dq, dk, dv, delta


def attn_bwd_rows(q, k, v, do, dtype: str, scale: float, causal: bool, rows):
    """dQ [n,D] and D_i [n] of sampled query rows (flat indices (b*H + h)*Sq + i)
    of 16-bit inputs, in float64; each row needs only its own scores."""
    q, k, v, do = _words(q), _words(k), _words(v), _words(do)
    B, H, Sq, Skv, D = _qkv_shapes(q, k, v, do)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    if rows.size and (rows.min() < 0 or rows.max() >= B * H * Sq):
        raise ValueError("row index out of range")
    dq = np.empty((rows.size, D))
    delta = np.empty((rows.size,))
    rc = _load().oracle_attn_bwd_rows(q.ctypes.data, k.ctypes.data, v.ctypes.data, do.ctypes.data,
                                      _DT[dtype], B, H, Sq, Skv, D, float(scale), int(bool(causal)),
                                      rows.ctypes.data, rows.size, dq.ctypes.data, delta.ctypes.data)
    if rc != 0:
        raise MemoryError("oracle scratch allocation failed")
    return dq, delta


def attn_bwd_keys(q, k, v, do, dtype: str, scale: float, causal: bool, keys):
    """dK [n,D] and dV [n,D] of sampled keys (flat indices (b*H + h)*Skv + j) of
    16-bit inputs, in float64 (cheap for keys few queries keep)."""
    q, k, v, do = _words(q), _words(k), _words(v), _words(do)
    B, H, Sq, Skv, D = _qkv_shapes(q, k, v, do)
    keys = np.ascontiguousarray(keys, dtype=np.int64)
    if keys.size and (keys.min() < 0 or keys.max() >= B * H * Skv):
        raise ValueError("key index out of range")
    dk = np.empty((keys.size, D))
    dv = np.empty((keys.size, D))
    rc = _load().oracle_attn_bwd_keys(q.ctypes.data, k.ctypes.data, v.ctypes.data, do.ctypes.data,
                                      _DT[dtype], B, H, Sq, Skv, D, float(scale), int(bool(causal)),
                                      keys.ctypes.data, keys.size, dk.ctypes.data, dv.ctypes.data)
    if rc != 0:
        raise MemoryError("oracle scratch allocation failed")
    return dk, dv
