"""GPU parity of attn_bwd against the fp64 oracle's backward.

The GPU forward supplies O and LSE (as a caller would); the oracle computes
dQ, dK, dV and D_i from Q, K, V, dO alone.  Gradients are compared as
max |x - x_ref| <= TOL_G[dtype] * max(1, max |x_ref|) per tensor; D_i as
|D - D_ref| <= TOL_G[dtype] * max(1, max |D_ref|).  Why these bounds: every
output is rounded once to 16 bits (u/2 of its own magnitude, u = 2^-11 for
fp16, 2^-8 for bf16); inside, P and dS are rounded to 16 bits before their
MFMAs and D_i uses the 16-bit O, each adding errors of u/2 relative per
term that partly cancel over the sums.  The measured worst case over these
cases is below 2u relative to the tensor's maximum; the bounds are 4u.
"""
import math

import numpy as np
import pytest

from exact_attention_52_amd import inputs

from gpu_util import to_dev, torch_dtype

pytestmark = pytest.mark.gpu

U = {"fp16": 2.0 ** -11, "bf16": 2.0 ** -8}
TOL_G = {k: 4 * u for k, u in U.items()}


@pytest.fixture(scope="module")
def ea():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_52_amd as m
    m._lib.load()
    return m


def gen(B, H, Sq, Skv, D, dtype, seed, mult=1.0):
    q, _, _ = inputs.gen_qkv(B, H, Sq, D, dtype, seed=seed, qk_mult=mult)
    _, k, v = inputs.gen_qkv(B, H, Skv, D, dtype, seed=seed + 1, qk_mult=mult)
    do, _, _ = inputs.gen_qkv(B, H, Sq, D, dtype, seed=seed + 2)
    return q, k, v, do


def f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def rel_err(x, ref):
    if ref.size == 0:
        return 0.0
    return float(np.abs(x - ref).max() / max(1.0, np.abs(ref).max()))


def run_case(ea, oracle_mod, B, H, Sq, Skv, D, dtype, causal, seed, mult=1.0, heads=None, scale=None):
    import torch
    print(f"bwd case B={B} H={H} Sq={Sq} Skv={Skv} D={D} {dtype} causal={causal} scale={scale}", flush=True)
    q, k, v, do = gen(B, H, Sq, Skv, D, dtype, seed, mult)
    if scale is None:
        scale = float(np.float32(1.0 / math.sqrt(D)))
    dq_, dk_, dv_, ddo = (to_dev(x, dtype) for x in (q, k, v, do))
    o, lse = ea.fwd(dq_, dk_, dv_, scale=scale, causal=causal)
    dq, dk, dv, delta = ea.bwd(dq_, dk_, dv_, o, lse, ddo, scale=scale, causal=causal)
    torch.cuda.synchronize()
    got = [f64(dq), f64(dk), f64(dv), delta.cpu().numpy().astype(np.float64)]
    if heads is not None:  # compare a subset of the b*H heads (each is independent)
        sel = lambda a: a.reshape((B * H,) + a.shape[2:])[heads][None]  # noqa: E731
        q, k, v, do = (sel(x) for x in (q, k, v, do))
        got = [sel(x) for x in got]
    ref = oracle_mod.attn_bwd(q, k, v, do, dtype, scale, causal)
    errs = [rel_err(a, b) for a, b in zip(got, ref)]
    print(f"  rel err dq {errs[0]:.2e} dk {errs[1]:.2e} dv {errs[2]:.2e} delta {errs[3]:.2e} "
          f"(tol {TOL_G[dtype]:.1e}; u {U[dtype]:.1e})", flush=True)
    for name, a in zip(("dq", "dk", "dv", "delta"), got):
        assert np.all(np.isfinite(a)), f"{name} not finite"
    for name, e in zip(("dq", "dk", "dv", "delta"), errs):
        assert e <= TOL_G[dtype], f"{name}: {e:.3e} > {TOL_G[dtype]:.3e}"
    return got, ref


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_square_ragged(ea, oracle_mod, D, dtype, causal):
    # several key and query tiles of every kernel plus a ragged tail
    run_case(ea, oracle_mod, 2, 2, 300, 300, D, dtype, causal, seed=D + 11)


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Sq,Skv", [(77, 333), (333, 77), (1, 200), (200, 1), (64, 64)])
def test_bwd_unequal_lengths(ea, oracle_mod, D, causal, Sq, Skv):
    dtype = "fp16" if (Sq + D) % 2 else "bf16"
    got, _ = run_case(ea, oracle_mod, 1, 3, Sq, Skv, D, dtype, causal, seed=Sq + 3 * Skv)
    if causal and Sq > Skv:  # queries with no key
        cut = Sq - Skv
        assert np.all(got[0][:, :, :cut] == 0.0) and np.all(got[3][:, :, :cut] == 0.0)


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_negative_scale(ea, oracle_mod, D, causal):
    # the page's sm_scale is a plain f32: a negative scale is valid
    dtype = "bf16" if D == 128 else "fp16"
    run_case(ea, oracle_mod, 1, 2, 211, 211, D, dtype, causal, seed=D + 17, scale=-0.09)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_bwd_peaky_scores(ea, oracle_mod, dtype):
    run_case(ea, oracle_mod, 1, 2, 257, 257, 128, dtype, True, seed=5, mult=2.0)


@pytest.mark.parametrize("D", [64, 128, 256])
def test_bwd_empty_sides(ea, D):
    import torch
    t = torch_dtype("bf16")
    q = torch.randn(1, 2, 40, D, device="cuda:0").to(t)
    none = torch.empty(1, 2, 0, D, device="cuda:0", dtype=t)
    # no keys: dQ = 0, D_i = 0 (O = 0, LSE = -inf from the forward)
    o, lse = ea.fwd(q, none, none)
    dq, dk, dv, delta = ea.bwd(q, none, none, o, lse, q, dq=torch.full_like(q, float("nan")),
                               delta=torch.full_like(lse, float("nan")))
    torch.cuda.synchronize()
    assert torch.all(dq == 0) and torch.all(delta == 0)
    # no queries: dK = dV = 0
    lse0 = torch.empty(1, 2, 0, device="cuda:0")
    dq, dk, dv, delta = ea.bwd(none, q, q, none, lse0, none, dk=torch.full_like(q, float("nan")),
                               dv=torch.full_like(q, float("nan")))
    torch.cuda.synchronize()
    assert torch.all(dk == 0) and torch.all(dv == 0)


def test_bwd_deterministic(ea):
    import torch
    q, k, v, do = gen(2, 4, 600, 600, 128, "bf16", seed=1)
    dev = [to_dev(x, "bf16") for x in (q, k, v, do)]
    o, lse = ea.fwd(*dev[:3], causal=True)
    a = ea.bwd(*dev[:3], o, lse, dev[3], causal=True)
    b = ea.bwd(*dev[:3], o, lse, dev[3], causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("wl,heads", [("c4_b2h16s4096d128_fp16_peaky", [0, 13, 31]),
                                      ("c3_b4h16s2048d128_bf16_causal", [0, 37, 63]),
                                      ("c2_b16h32s1024d64_fp16_causal", [0, 255, 511]),
                                      ("c5_b1h8s8192d256_bf16_causal", [3])])
def test_bwd_full_size(ea, oracle_mod, wl, heads):
    B, H, S, D, dtype, causal, mult = inputs.WORKLOADS[wl]
    run_case(ea, oracle_mod, B, H, S, S, D, dtype, causal, seed=0, mult=mult, heads=heads)


def as_layout(t, layout):
    import torch
    B, H, S, D = t.shape
    if layout == "bshd":
        return t.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    if layout == "padded":
        buf = torch.zeros((B, H, S, D + 8), dtype=t.dtype, device=t.device)
        buf[..., :D] = t
        return buf[..., :D]
    return t


@pytest.mark.parametrize("D,dtype,causal", [(64, "fp16", True), (128, "bf16", False), (128, "fp16", True),
                                            (256, "bf16", True)])
@pytest.mark.parametrize("layout", ["bshd", "padded"])
def test_bwd_strided_equals_contiguous_bitwise(ea, D, dtype, causal, layout):
    # the layout changes the addresses, not the arithmetic
    import torch
    q, k, v, do = gen(2, 3, 300, 300, D, dtype, seed=D + 1)
    dev = [to_dev(x, dtype) for x in (q, k, v, do)]
    o, lse = ea.fwd(*dev[:3], causal=causal)
    ref = ea.bwd(*dev[:3], o, lse, dev[3], causal=causal)
    ins = [as_layout(t, layout) for t in (*dev[:3], o, dev[3])]
    outs = [as_layout(torch.full_like(t, float("nan")), layout) for t in dev[:3]]
    got = ea.bwd(*ins[:4], lse, ins[4], causal=causal, dq=outs[0], dk=outs[1], dv=outs[2])
    torch.cuda.synchronize()
    for a, b in zip(got, ref):
        assert torch.equal(a, b)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_strided_unequal_lengths_vs_oracle(ea, oracle_mod, causal):
    import torch
    D, dtype = 128, "fp16"
    q, k, v, do = gen(1, 2, 150, 333, D, dtype, seed=4)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    dev = [as_layout(to_dev(x, dtype), "bshd") for x in (q, k, v, do)]
    o, lse = ea.fwd(*dev[:3], scale=scale, causal=causal)
    got = ea.bwd(*dev[:3], o, lse, dev[3], scale=scale, causal=causal)
    torch.cuda.synchronize()
    ref = oracle_mod.attn_bwd(q, k, v, do, dtype, scale, causal)
    for name, a, r in zip(("dq", "dk", "dv", "delta"), got, ref):
        e = rel_err(a.float().cpu().numpy().astype(np.float64), r)
        assert e <= TOL_G[dtype], f"{name}: {e:.3e}"


@pytest.mark.parametrize("D,dtype,causal", [(64, "bf16", True), (128, "fp16", False), (256, "fp16", True)])
def test_autograd_wrapper(ea, oracle_mod, D, dtype, causal):
    # attention() through torch.autograd gives the oracle's gradients
    import torch
    q, k, v, do = gen(1, 2, 130, 200, D, dtype, seed=D + 9)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    dev = [to_dev(x, dtype).requires_grad_(True) for x in (q, k, v)]
    out = ea.attention(*dev, scale=scale, causal=causal)
    out.backward(to_dev(do, dtype))
    torch.cuda.synchronize()
    dq_ref, dk_ref, dv_ref, _ = oracle_mod.attn_bwd(q, k, v, do, dtype, scale, causal)
    for name, t, r in zip(("dq", "dk", "dv"), dev, (dq_ref, dk_ref, dv_ref)):
        e = rel_err(t.grad.float().cpu().numpy().astype(np.float64), r)
        assert e <= TOL_G[dtype], f"{name}: {e:.3e}"
