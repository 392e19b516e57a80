"""Rows past the end of a tensor read as zero.

Every tensor the kernels stream through LDS (K and V in the forward and in
the backward's dQ kernel; Q and dO in the backward's dK/dV kernel) is placed
at the very end of its data inside a larger allocation whose remaining
elements are NaN, and the key and query lengths leave the last tile ragged.
The copies of that tile must read the rows past the end as 0 (the buffer
descriptor's range check), never the NaN that follows: a NaN row of V or dO
would reach the outputs through a zero weight (0 * NaN = NaN).  The NaN
region lies inside the test's own allocation, so an over-read shows up as a
non-finite output, not as a memory fault.
"""
import math

import numpy as np
import pytest

from exact_attention_52_amd import inputs

from gpu_util import TOL_LSE, TOL_O, errors, o_to_f64, to_dev

pytestmark = pytest.mark.gpu

PAD = 1 << 17  # NaN elements after each tensor (256 KiB), more than any tile


@pytest.fixture(scope="module")
def ea():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_52_amd as m
    m._lib.load()
    return m


def nan_tailed(words, dtype):
    """The tensor on the device as the first elements of a NaN-filled buffer."""
    import torch
    t = to_dev(words, dtype)
    buf = torch.full((t.numel() + PAD,), float("nan"), dtype=t.dtype, device=t.device)
    buf[: t.numel()].copy_(t.reshape(-1))
    view = buf[: t.numel()].view(t.shape)
    assert view.data_ptr() == buf.data_ptr()
    return view, buf


# (D, S): S leaves the last key tile (64 keys at D = 64 and 256, 128 at
# D = 128) with a few rows, and the last query tile ragged too
CASES = [(64, 130), (128, 130), (128, 300), (256, 70), (256, 200)]


@pytest.mark.parametrize("D,S", CASES)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_forward_reads_zero_past_the_end(ea, D, S, causal, dtype):
    import torch
    import oracle
    B, H = 1, 2
    print(f"tail guard fwd D={D} S={S} causal={causal} {dtype}", flush=True)
    q, k, v = inputs.gen_qkv(B, H, S, D, dtype, seed=31)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    dq = to_dev(q, dtype)
    dk, _bk = nan_tailed(k, dtype)
    dv, _bv = nan_tailed(v, dtype)
    o, lse = ea.fwd(dq, dk, dv, scale=scale, causal=causal)
    torch.cuda.synchronize()
    og, lg = o_to_f64(o), lse.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(og)) and np.all(np.isfinite(lg))
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, dtype, scale, causal)
    eo, el = errors(og, lg, o_ref, lse_ref)
    assert eo <= TOL_O[dtype] and el <= TOL_LSE, (eo, el)


U = {"fp16": 2.0 ** -11, "bf16": 2.0 ** -8}


@pytest.mark.parametrize("D,S", CASES)
@pytest.mark.parametrize("causal", [False, True])
def test_backward_reads_zero_past_the_end(ea, D, S, causal):
    import torch
    import oracle
    B, H, dtype = 1, 2, "fp16"
    print(f"tail guard bwd D={D} S={S} causal={causal}", flush=True)
    q, k, v = inputs.gen_qkv(B, H, S, D, dtype, seed=32)
    do, _, _ = inputs.gen_qkv(B, H, S, D, dtype, seed=33)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    tq, _bq = nan_tailed(q, dtype)
    tk, _bk = nan_tailed(k, dtype)
    tv, _bv = nan_tailed(v, dtype)
    tdo, _bdo = nan_tailed(do, dtype)
    o, lse = ea.fwd(tq, tk, tv, scale=scale, causal=causal)
    got = ea.bwd(tq, tk, tv, o, lse, tdo, scale=scale, causal=causal)
    torch.cuda.synchronize()
    ref = oracle.attn_bwd(q, k, v, do, dtype, scale, causal)
    for name, g, r in zip(("dq", "dk", "dv", "delta"), got, ref):
        a = g.float().cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(a)), f"{name} not finite"
        e = float(np.abs(a - r).max() / max(1.0, np.abs(r).max()))
        assert e <= 4 * U[dtype], f"{name}: {e:.3e}"
