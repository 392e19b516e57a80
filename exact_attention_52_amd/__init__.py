"""Exact attention forward for MI355X (gfx950).

``fwd(q, k, v, scale=None, causal=False)`` returns ``(o, lse)`` for fp16/bf16
CUDA tensors q [B,H,Sq,D] and k, v [B,H,Skv,D] (any strides with the last
dimension contiguous): O = softmax(scale * Q K^T [causal]) V and the
natural-log LSE per row (fp32).  ``bwd(q, k, v, o, lse, do, ...)`` returns
``(dq, dk, dv, delta)``, the gradients for a given dO (any such strides);
``attention(q, k, v, scale, causal)`` wraps both as a torch.autograd function.
PyTorch only provides device memory and the
stream; the computation is the libattn.so gfx950 kernel behind the C ABI of
include/attn.h (the unfused comparator ``fwd_unfused``: libattn_unfused.so,
include/attn_unfused.h).  ``inputs`` holds the seeded synthetic-input generator.
"""
from __future__ import annotations

import math

from . import _lib
from ._lib import ATTN_BF16, ATTN_F16, AttnError  # noqa: F401

__all__ = ["attention", "fwd", "bwd", "fwd_unfused", "fwd_variant", "attn_fwd", "attn_fwd_strided", "attn_fwd_variant",
           "attn_bwd", "attn_bwd_strided", "attn_bwd_noalloc", "attn_fwd_unfused",
           "attn_fwd_unfused_workspace_bytes", "attn_fwd_plan", "attn_fwd_workgroup_tile", "AttnError"]

attn_fwd = _lib.attn_fwd
attn_fwd_strided = _lib.attn_fwd_strided
attn_bwd = _lib.attn_bwd
attn_bwd_strided = _lib.attn_bwd_strided
attn_bwd_noalloc = _lib.attn_bwd_noalloc
attn_fwd_variant = _lib.attn_fwd_variant
attn_fwd_unfused = _lib.attn_fwd_unfused
attn_fwd_unfused_workspace_bytes = _lib.attn_fwd_unfused_workspace_bytes
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

    q: CUDA tensor [B,H,Sq,D]; k, v: [B,H,Skv,D]; one dtype (fp16 or bf16);
    any strides with the last dimension contiguous (e.g. views of [B,S,H,D]).
    Causal keeps key j for query i iff j <= i + Skv - Sq.  scale defaults to
    1/sqrt(D).  out ([B,H,Sq,D], input dtype, any such strides) and lse
    (contiguous fp32 [B,H,Sq]) may be passed preallocated.  Returns (o, lse).
    """
    import torch
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D: [B,H,Sq,D], [B,H,Skv,D], [B,H,Skv,D]")
    B, H, Sq, D = q.shape
    Skv = k.shape[2]
    if k.shape != (B, H, Skv, D) or v.shape != k.shape:
        raise ValueError("k and v must be [B,H,Skv,D] with q's B, H and D")
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k, v must be GPU tensors")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    dt = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, H, Sq, D), dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must be [B,H,Sq,D] in the input dtype")
    if lse.shape != (B, H, Sq) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B,H,Sq] tensor")
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        if D > 1 and t.stride(3) != 1:
            raise ValueError(f"{name} must have its last dimension contiguous")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    plain = Sq == Skv and all(t.is_contiguous() for t in (q, k, v, out))
    with torch.cuda.device(q.device):
        if plain:
            st = _lib.attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                               lse.data_ptr(), B, H, Sq, D, scale, causal, dt, stream.cuda_stream)
        else:
            st = _lib.attn_fwd_strided(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                       lse.data_ptr(), B, H, Sq, Skv, D, q.stride()[:3], k.stride()[:3],
                                       v.stride()[:3], out.stride()[:3], scale, causal, dt,
                                       stream.cuda_stream)
    _lib.check(st)
    return out, lse


def bwd(q, k, v, o, lse, do, scale=None, causal=False, dq=None, dk=None, dv=None, delta=None,
        stream=None):
    """Gradients of ``fwd`` for the output gradient ``do``.

    q, o, do: [B,H,Sq,D]; k, v: [B,H,Skv,D]; one dtype (fp16 or bf16); any
    strides with the last dimension contiguous (e.g. views of [B,S,H,D]);
    lse: contiguous fp32 [B,H,Sq], with o and lse from ``fwd`` on the same
    inputs.  Returns (dq, dk, dv, delta): dq [B,H,Sq,D], dk, dv [B,H,Skv,D] in
    the input dtype (fresh contiguous tensors unless passed in, with any such
    strides) and delta = rowsum(do * o), contiguous fp32 [B,H,Sq].
    """
    import torch
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        if t.dim() != 4 or not t.is_cuda:
            raise ValueError(f"{name} must be a 4-D GPU tensor")
        if t.dtype != q.dtype:
            raise TypeError("q, k, v, o, do must share one dtype")
    B, H, Sq, D = q.shape
    Skv = k.shape[2]
    if k.shape != (B, H, Skv, D) or v.shape != k.shape:
        raise ValueError("k and v must be [B,H,Skv,D] with q's B, H and D")
    if o.shape != q.shape or do.shape != q.shape:
        raise ValueError("o and do must have q's shape")
    if lse.shape != (B, H, Sq) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B,H,Sq] tensor")
    dt = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    dq = torch.empty_like(q, memory_format=torch.contiguous_format) if dq is None else dq
    dk = torch.empty_like(k, memory_format=torch.contiguous_format) if dk is None else dk
    dv = torch.empty_like(v, memory_format=torch.contiguous_format) if dv is None else dv
    delta = torch.empty_like(lse) if delta is None else delta
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if t.shape != ref.shape or t.dtype != ref.dtype:
            raise ValueError(f"{name} must have the shape and dtype of its input")
    if delta.shape != lse.shape or delta.dtype != torch.float32 or not delta.is_contiguous():
        raise ValueError("delta must be a contiguous float32 [B,H,Sq] tensor")
    tensors = (q, k, v, o, do, dq, dk, dv)
    for name, t in zip(("q", "k", "v", "o", "do", "dq", "dk", "dv"), tensors):
        if D > 1 and t.stride(3) != 1:
            raise ValueError(f"{name} must have its last dimension contiguous")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    ptrs = [t.data_ptr() for t in (q, k, v, o)] + [lse.data_ptr(), do.data_ptr()] + \
        [t.data_ptr() for t in (dq, dk, dv)] + [delta.data_ptr()]
    with torch.cuda.device(q.device):
        if all(t.is_contiguous() for t in tensors):
            st = _lib.attn_bwd(*ptrs, B, H, Sq, Skv, D, scale, causal, dt, stream.cuda_stream)
        else:
            st = _lib.attn_bwd_strided(*ptrs, B, H, Sq, Skv, D, [t.stride()[:3] for t in tensors], scale,
                                       causal, dt, stream.cuda_stream)
    _lib.check(st)
    return dq, dk, dv, delta


def fwd_unfused(q, k, v, scale=None, causal=False, out=None, lse=None, workspace=None, stream=None):
    """The unfused comparator of ``fwd``: S = scale Q K^T in HBM (fp32), a row
    softmax writing P, then O = P V.  q, k, v contiguous [B,H,S,D] of one
    dtype.  ``workspace`` (a uint8 CUDA tensor of at least
    ``attn_fwd_unfused_workspace_bytes(B, H, S, D)`` bytes) may be passed in.
    Returns (o, lse)."""
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dim() != 4 or not t.is_cuda or not t.is_contiguous() or t.dtype != q.dtype:
            raise ValueError(f"{name} must be a contiguous 4-D GPU tensor of q's dtype")
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one [B,H,S,D] shape")
    B, H, S, D = q.shape
    dt = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device) if lse is None else lse
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be contiguous [B,H,S,D] in the input dtype")
    if lse.shape != (B, H, S) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B,H,S] tensor")
    need = _lib.attn_fwd_unfused_workspace_bytes(B, H, S, D)
    if need < 0:
        raise ValueError("shape too large for the unfused path")
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    with torch.cuda.device(q.device):
        st = _lib.attn_fwd_unfused(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                   workspace.data_ptr(), workspace.numel() * workspace.element_size(), B, H, S,
                                   D, scale, causal, dt, stream.cuda_stream)
    _lib.check_unfused(st)
    return out, lse


def fwd_variant(q, k, v, variant, scale=None, causal=False, out=None, lse=None, stream=None):
    """``fwd`` on contiguous [B,H,S,D] tensors with copy schedule ``variant``
    (0: shipped; 1/2/3: K/V LDS stages; 4: 2 stages plus a producer wave;
    5/6: the shipped tile shape with 1 or 2 stages and no ping-pong).
    Returns (o, lse)."""
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dim() != 4 or not t.is_cuda or not t.is_contiguous() or t.dtype != q.dtype or t.shape != q.shape:
            raise ValueError(f"{name} must be a contiguous [B,H,S,D] GPU tensor like q")
    B, H, S, D = q.shape
    dt = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device) if lse is None else lse
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be contiguous [B,H,S,D] in the input dtype")
    if lse.shape != (B, H, S) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B,H,S] tensor")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    with torch.cuda.device(q.device):
        st = _lib.attn_fwd_variant(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                   B, H, S, D, scale, causal, dt, int(variant), stream.cuda_stream)
    _lib.check(st)
    return out, lse


def _autograd_function():
    import torch

    class _Attention(torch.autograd.Function):
        """O = attention(q, k, v) with the library's forward and backward kernels;
        O and LSE are saved for the backward (the page's recomputation from the
        saved log-sum-exp)."""

        @staticmethod
        def forward(ctx, q, k, v, scale, causal):
            o, lse = fwd(q, k, v, scale=scale, causal=causal)
            ctx.save_for_backward(q, k, v, o, lse)
            ctx.scale, ctx.causal = scale, causal
            return o

        @staticmethod
        def backward(ctx, do):
            q, k, v, o, lse = ctx.saved_tensors
            dq, dk, dv, _ = bwd(q, k, v, o, lse, do.contiguous() if do.stride(-1) != 1 else do,
                                scale=ctx.scale, causal=ctx.causal)
            return dq, dk, dv, None, None

    return _Attention


_ATTENTION = None


def attention(q, k, v, scale=None, causal=False):
    """Differentiable exact attention: ``fwd`` forward, ``bwd`` backward
    (torch.autograd).  q [B,H,Sq,D], k, v [B,H,Skv,D], fp16 or bf16 CUDA
    tensors with the last dimension contiguous.  Returns O."""
    global _ATTENTION
    if _ATTENTION is None:
        _ATTENTION = _autograd_function()
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    return _ATTENTION.apply(q, k, v, float(scale), bool(causal))
