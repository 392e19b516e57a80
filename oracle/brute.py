"""TEST INFRASTRUCTURE ONLY: pure-Python brute-force attention for tiny shapes.

An independent second implementation of the definition used by the C oracle
(docs.rs page "oxicuda-dnn 0.1.8, src/attn/flash_attn/hopper.rs", doc comment
of FlashAttention3Plan::generate_forward: scores Q K^T times the softmax scale,
causal positions after the query removed, softmax, times V, plus the
log-sum-exp of the scaled scores).  It decodes the 16-bit words with the
standard library's ``struct`` module and sums with ``math.fsum`` (correctly
rounded sums), so it shares nothing with the C code beyond the definition.
"""
from __future__ import annotations

import math
import struct


def decode(word: int, dtype: str) -> float:
    if dtype == "fp16":
        return struct.unpack("<e", struct.pack("<H", word))[0]
    if dtype == "bf16":
        return struct.unpack("<f", struct.pack("<I", word << 16))[0]
    raise ValueError(dtype)


def attention(q, k, v, dtype: str, scale: float, causal: bool):
    """q: nested lists [B][H][Sq][D], k, v: [B][H][Skv][D] of 16-bit words.

    Causal keeps key j for query i iff j <= i + Skv - Sq (the last query sees
    the last key); a query with no key gets O = 0 and LSE = -inf.
    Returns (O, LSE) as nested lists of Python floats.
    """
    B, H, Sq, D = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Skv = len(k[0][0])
    O = [[[[0.0] * D for _ in range(Sq)] for _ in range(H)] for _ in range(B)]
    L = [[[0.0] * Sq for _ in range(H)] for _ in range(B)]
    for b in range(B):
        for h in range(H):
            Q = [[decode(w, dtype) for w in row] for row in q[b][h]]
            K = [[decode(w, dtype) for w in row] for row in k[b][h]]
            V = [[decode(w, dtype) for w in row] for row in v[b][h]]
            for i in range(Sq):
                keys = range(max(0, min(Skv, i + 1 + Skv - Sq))) if causal else range(Skv)
                if not keys:
                    L[b][h][i] = -math.inf
                    continue
                s = {j: scale * math.fsum(Q[i][d] * K[j][d] for d in range(D))
                     for j in keys}
                m = max(s.values())
                w = {j: math.exp(s[j] - m) for j in keys}
                l = math.fsum(w.values())
                for d in range(D):
                    O[b][h][i][d] = math.fsum(w[j] * V[j][d] for j in keys) / l
                L[b][h][i] = m + math.log(l)
    return O, L
