"""Seeded synthetic inputs for the attention forward: Philox4x32-10 + Box-Muller.

This module holds no attention arithmetic. It turns (seed, tensor id, shape,
dtype, multiplier) into the exact 16-bit words that both the GPU path and the
CPU oracle consume, so the two sides see identical bytes.

Definition (written from the published descriptions, not from any library):

* Counter-based generator: Philox4x32 with 10 rounds (Salmon, Moraes, Dror,
  Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC'11). One round maps a
  counter (c0,c1,c2,c3) under key (k0,k1) to
  (hi(M1*c2) ^ c1 ^ k0, lo(M1*c2), hi(M0*c0) ^ c3 ^ k1, lo(M0*c0)) with
  M0 = 0xD2511F53, M1 = 0xCD9E8D57; between rounds the key is bumped by the
  Weyl constants (0x9E3779B9, 0xBB67AE85).
* Stream layout: key = (seed & 0xFFFFFFFF, tensor_id); the counter for the
  group of four elements 4n..4n+3 of the C-order flattened tensor is
  (n & 0xFFFFFFFF, n >> 32, 0, 0). Any slice can therefore be regenerated on
  its own.
* Uniforms: u = (x + 0.5) / 2**32 for each 32-bit output word x, so u lies in
  the open interval (0, 1).
* Normals: Box-Muller (1958) in float64 on the pairs (u0,u1) and (u2,u3):
  r = sqrt(-2 ln ua), z_a = r cos(2 pi ub), z_b = r sin(2 pi ub).
* The normals are multiplied by ``mult`` (exact for powers of two), then
  rounded to nearest-even: straight to fp16, or to fp32 and then to bf16.

Tensor ids: Q = 0, K = 1, V = 2.
"""
from __future__ import annotations

import hashlib

import numpy as np

PHILOX_M0 = np.uint64(0xD2511F53)
PHILOX_M1 = np.uint64(0xCD9E8D57)
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
MASK32 = np.uint64(0xFFFFFFFF)

TENSOR_Q, TENSOR_K, TENSOR_V = 0, 1, 2
DTYPES = ("fp16", "bf16")


def philox4x32_10(ctr, key):
    """Philox4x32-10 on arrays.

    ctr: tuple of four uint32-valued arrays (or scalars); key: (k0, k1) ints.
    Returns a tuple of four uint32 numpy arrays.
    """
    c0, c1, c2, c3 = (np.asarray(c, dtype=np.uint64) for c in ctr)
    k0, k1 = int(key[0]) & 0xFFFFFFFF, int(key[1]) & 0xFFFFFFFF
    for rnd in range(10):
        if rnd:
            k0 = (k0 + PHILOX_W0) & 0xFFFFFFFF
            k1 = (k1 + PHILOX_W1) & 0xFFFFFFFF
        p0 = PHILOX_M0 * c0
        p1 = PHILOX_M1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & MASK32
        c0, c1, c2, c3 = (hi1 ^ c1 ^ np.uint64(k0), lo1,
                          hi0 ^ c3 ^ np.uint64(k1), lo0)
    return tuple(c.astype(np.uint32) for c in (c0, c1, c2, c3))


def normals(seed: int, tensor_id: int, n_elems: int, start: int = 0) -> np.ndarray:
    """float64 N(0,1) values for flat element indices [start, start+n_elems)."""
    if n_elems <= 0:
        return np.zeros(0, dtype=np.float64)
    g0 = start // 4
    g1 = (start + n_elems + 3) // 4
    n = np.arange(g0, g1, dtype=np.uint64)
    x0, x1, x2, x3 = philox4x32_10(
        (n & MASK32, n >> np.uint64(32), np.zeros_like(n), np.zeros_like(n)),
        (seed, tensor_id))
    inv = 1.0 / 4294967296.0
    u = [(x.astype(np.float64) + 0.5) * inv for x in (x0, x1, x2, x3)]
    out = np.empty((g1 - g0, 4), dtype=np.float64)
    for col, (ua, ub) in enumerate(((u[0], u[1]), (u[2], u[3]))):
        r = np.sqrt(-2.0 * np.log(ua))
        th = 2.0 * np.pi * ub
        out[:, 2 * col] = r * np.cos(th)
        out[:, 2 * col + 1] = r * np.sin(th)
    flat = out.reshape(-1)
    off = start - 4 * g0
    return flat[off:off + n_elems]


def round_to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to nearest-even 16-bit words (uint16)."""
    if dtype == "fp16":
        return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        f = np.asarray(x, dtype=np.float64).astype(np.float32)
        b = f.view(np.uint32).astype(np.uint64)
        lsb = (b >> np.uint64(16)) & np.uint64(1)
        r = (b + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
        return r.astype(np.uint16)
    raise ValueError(f"dtype must be one of {DTYPES}, got {dtype!r}")


def gen_tensor(seed: int, tensor_id: int, shape, dtype: str, mult: float = 1.0) -> np.ndarray:
    """The 16-bit words (uint16, C order, ``shape``) of one generated tensor."""
    n = int(np.prod(shape)) if len(shape) else 1
    z = normals(seed, tensor_id, n)
    if mult != 1.0:
        z = z * mult
    return round_to_bits(z, dtype).reshape(shape)


def gen_qkv(B: int, H: int, S: int, D: int, dtype: str, seed: int = 0,
            qk_mult: float = 1.0):
    """Q, K, V as uint16 arrays of shape [B,H,S,D] (Q,K optionally scaled)."""
    shape = (B, H, S, D)
    q = gen_tensor(seed, TENSOR_Q, shape, dtype, qk_mult)
    k = gen_tensor(seed, TENSOR_K, shape, dtype, qk_mult)
    v = gen_tensor(seed, TENSOR_V, shape, dtype, 1.0)
    return q, k, v


def bits_to_float(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Widen 16-bit words to float32 (exact) for inspection and statistics."""
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == "fp16":
        return bits.view(np.float16).astype(np.float32)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    raise ValueError(dtype)


def sha256_hex(arr: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(arr).tobytes()).hexdigest()


# The five workloads: (name, B, H, S, D, dtype, causal, qk_mult). scale = 1/sqrt(D).
WORKLOADS = {
    "c1_b1h2s128d64_fp16": (1, 2, 128, 64, "fp16", False, 1.0),
    "c2_b16h32s1024d64_fp16_causal": (16, 32, 1024, 64, "fp16", True, 1.0),
    "c3_b4h16s2048d128_bf16_causal": (4, 16, 2048, 128, "bf16", True, 1.0),
    "c4_b2h16s4096d128_fp16_peaky": (2, 16, 4096, 128, "fp16", False, 2.0),
    "c5_b1h8s8192d256_bf16_causal": (1, 8, 8192, 256, "bf16", True, 1.0),
}
