"""Exact attention forward for MI355X (gfx950).

``fwd(q, k, v, scale=None, causal=False)`` returns ``(o, lse)`` for contiguous
[B,H,S,D] fp16/bf16 CUDA tensors: O = softmax(scale * Q K^T [causal]) V and
the natural-log LSE per row (fp32).  PyTorch only provides device memory and
the stream; the computation is the libattn.so gfx950 kernel behind the C ABI
of include/attn.h.  ``inputs`` holds the seeded synthetic-input generator.
"""
from __future__ import annotations

import math

from . import _lib
from ._lib import ATTN_BF16, ATTN_F16, AttnError  # noqa: F401

__all__ = ["fwd", "attn_fwd", "attn_fwd_plan", "attn_fwd_workgroup_tile", "AttnError"]

attn_fwd = _lib.attn_fwd
attn_fwd_plan = _lib.attn_fwd_plan
attn_fwd_workgroup_tile = _lib.attn_fwd_workgroup_tile


def _dtype_code(t):
    import torch
    if t.dtype == torch.float16:
        return ATTN_F16
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    raise TypeError(f"q, k, v must be float16 or bfloat16, got {t.dtype}")


def fwd(q, k, v, scale=None, causal=False, out=None, lse=None, stream=None):
    """Run the attention forward on the current (or given) stream.

    q, k, v: contiguous CUDA tensors [B,H,S,D] of one dtype (fp16 or bf16).
    scale defaults to 1/sqrt(D).  out / lse may be passed preallocated.
    Returns (o, lse) with o [B,H,S,D] in the input dtype and lse [B,H,S] fp32.
    """
    import torch
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must all be [B,H,S,D] with one shape")
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k, v must be GPU tensors")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    dt = _dtype_code(q)
    B, H, S, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like q")
    if lse.shape != (B, H, S) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B,H,S] tensor")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    with torch.cuda.device(q.device):
        st = _lib.attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                           lse.data_ptr(), B, H, S, D, scale, causal, dt, stream.cuda_stream)
    _lib.check(st)
    return out, lse
