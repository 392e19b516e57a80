"""Largest sizes: long sequences (one head near the 32-bit per-head offset
range the kernels use), a grid of 2^18 heads, the backward at S = 2^17
(2^16 for D = 256) and over 2^16 short heads, tensors past 4 GiB (forward
and backward), checked on outputs the oracle computes one by one (sampled
query rows, sampled keys few queries see, sampled heads) and on identities
that hold at any size.

Inputs here are seeded standard normals from numpy's PCG64 (not the Philox
generator of the workloads: at 2^28 elements per tensor that would take
minutes), rounded to 16 bits by the shared input module.
"""
import math

import numpy as np
import pytest

from exact_attention_52_amd import inputs

from gpu_util import TOL_LSE, TOL_O, errors, o_to_f64, to_dev

pytestmark = pytest.mark.gpu

U = {"fp16": 2.0 ** -11, "bf16": 2.0 ** -8}


@pytest.fixture(scope="module")
def ea():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_52_amd as m
    m._lib.load()
    return m


def words(shape, dtype, seed, mult=1.0):
    x = np.random.default_rng(seed).standard_normal(shape, dtype=np.float32)
    if mult != 1.0:
        x *= mult
    return inputs.round_to_bits(x, dtype).reshape(shape)


@pytest.mark.parametrize("B,H,S,D,dtype,causal", [
    (1, 1, 1 << 22, 64, "fp16", True),     # 512 MiB per tensor, one head
    (1, 1, 1 << 20, 128, "bf16", False),
    (1, 1, 1 << 19, 256, "bf16", True),
    (256, 1024, 5, 64, "fp16", False),     # 2^18 heads: 2^18 workgroups
])
def test_forward_largest_sizes(ea, oracle_mod, B, H, S, D, dtype, causal):
    import torch
    print(f"large fwd B={B} H={H} S={S} D={D} {dtype} causal={causal}", flush=True)
    q, k, v = (words((B, H, S, D), dtype, seed=S + i) for i in range(3))
    scale = float(np.float32(1.0 / math.sqrt(D)))
    o, lse = ea.fwd(*(to_dev(x, dtype) for x in (q, k, v)), scale=scale, causal=causal)
    torch.cuda.synchronize()
    n = B * H * S
    rows = np.unique(np.concatenate([[0, n - 1, S - 1, n // 2],
                                     np.random.default_rng(7).integers(0, n, 24)]))
    o_ref, lse_ref = oracle_mod.attn_fwd(q, k, v, dtype, scale, causal, rows=rows)
    og = o.view(-1, D)[torch.from_numpy(rows).to(o.device)]
    lg = lse.view(-1)[torch.from_numpy(rows).to(o.device)]
    eo, el = errors(o_to_f64(og), lg.cpu().numpy().astype(np.float64), o_ref, lse_ref)
    assert eo <= TOL_O[dtype], f"max|dO| {eo:.3e}"
    assert el <= TOL_LSE, f"max dLSE {el:.3e}"


@pytest.mark.parametrize("D,dtype,S", [(128, "fp16", 1 << 17), (64, "bf16", 1 << 17), (256, "bf16", 1 << 16)])
def test_backward_long_causal_sequence(ea, oracle_mod, D, dtype, S):
    import torch
    print(f"large bwd S={S} D={D} {dtype} causal", flush=True)
    q, k, v, do = (words((1, 1, S, D), dtype, seed=11 + i) for i in range(4))
    scale = float(np.float32(1.0 / math.sqrt(D)))
    dev = [to_dev(x, dtype) for x in (q, k, v, do)]
    o, lse = ea.fwd(*dev[:3], scale=scale, causal=True)
    dq, dk, dv, delta = ea.bwd(*dev[:3], o, lse, dev[3], scale=scale, causal=True)
    torch.cuda.synchronize()
    tol = 4 * U[dtype]

    # sampled query rows: dQ_i and D_i need only row i's scores
    rows = np.array([0, 1, 777, S // 2, S - 2, S - 1])
    dq_ref, delta_ref = oracle_mod.attn_bwd_rows(q, k, v, do, dtype, scale, True, rows)
    sel = torch.from_numpy(rows).to(dq.device)
    dq_g = dq.view(-1, D)[sel].float().cpu().numpy().astype(np.float64)
    de_g = delta.view(-1)[sel].cpu().numpy().astype(np.float64)
    assert np.abs(dq_g - dq_ref).max() <= tol * max(1.0, np.abs(dq_ref).max())
    assert np.abs(de_g - delta_ref).max() <= tol * max(1.0, np.abs(delta_ref).max())

    # the last keys: few queries keep them, so the oracle computes them directly
    keys = np.arange(S - 12, S)
    dk_ref, dv_ref = oracle_mod.attn_bwd_keys(q, k, v, do, dtype, scale, True, keys)
    selk = torch.from_numpy(keys).to(dk.device)
    dk_g = dk.view(-1, D)[selk].float().cpu().numpy().astype(np.float64)
    dv_g = dv.view(-1, D)[selk].float().cpu().numpy().astype(np.float64)
    assert np.abs(dk_g - dk_ref).max() <= tol * max(1.0, np.abs(dk_ref).max())
    assert np.abs(dv_g - dv_ref).max() <= tol * max(1.0, np.abs(dv_ref).max())

    # identities at full size: every row of dS sums to 0, so the dK rows sum
    # to 0; the dV rows sum to the dO rows (every query sees a key).  Each of
    # the S rounded rows carries at most ~2u of its own size, so the sums are
    # compared against u times the sum of magnitudes.
    dk64 = dk.double().sum(dim=2)[0, 0].cpu().numpy()
    mag = dk.double().abs().sum(dim=2)[0, 0].cpu().numpy()
    assert np.all(np.abs(dk64) <= 2 * U[dtype] * mag + 1e-6), (np.abs(dk64) / mag).max()
    dv_sum = dv.double().sum(dim=2)[0, 0].cpu().numpy()
    do_sum = inputs.bits_to_float(do, dtype).sum(axis=2)[0, 0]
    dv_mag = dv.double().abs().sum(dim=2)[0, 0].cpu().numpy()
    assert np.all(np.abs(dv_sum - do_sum) <= 2 * U[dtype] * dv_mag + 1e-6), \
        (np.abs(dv_sum - do_sum) / dv_mag).max()


def test_backward_many_heads(ea, oracle_mod):
    # 2^16 heads of 7 rows: the grid and head arithmetic at scale, checked in full
    import torch
    B, H, S, D, dtype = 64, 1024, 7, 64, "fp16"
    q, k, v, do = (words((B, H, S, D), dtype, seed=21 + i) for i in range(4))
    scale = float(np.float32(1.0 / math.sqrt(D)))
    dev = [to_dev(x, dtype) for x in (q, k, v, do)]
    o, lse = ea.fwd(*dev[:3], scale=scale, causal=False)
    got = ea.bwd(*dev[:3], o, lse, dev[3], scale=scale, causal=False)
    torch.cuda.synchronize()
    ref = oracle_mod.attn_bwd(q, k, v, do, dtype, scale, False)
    tol = 4 * U[dtype]
    for name, g, r in zip(("dq", "dk", "dv", "delta"), got, ref):
        g = g.float().cpu().numpy().astype(np.float64)
        assert np.abs(g - r).max() <= tol * max(1.0, np.abs(r).max()), name


@pytest.mark.parametrize("D,dtype,causal", [(64, "fp16", True), (128, "fp16", False), (256, "bf16", True)])
def test_tensors_past_4gib(ea, oracle_mod, D, dtype, causal):
    # Every tensor larger than 2^32 bytes (heads of 256 rows, enough of them
    # that the last ones start past 4 GiB): forward and backward, checked in
    # full on sampled heads on both sides of the 4 GiB mark.  The inputs are
    # seeded normals drawn on the device by torch (host generation of 2^31
    # elements per tensor would take minutes); the sampled heads' words are
    # copied back for the oracle.
    import torch
    S = 256
    head_bytes = S * D * 2
    H = (1 << 32) // head_bytes + 37
    B = 1
    print(f"past 4 GiB: B={B} H={H} S={S} D={D} {dtype} causal={causal}", flush=True)
    tdt = torch.float16 if dtype == "fp16" else torch.bfloat16
    g = torch.Generator(device="cuda:0").manual_seed(4321 + D)
    q, k, v, do = (torch.randn((B, H, S, D), generator=g, device="cuda:0", dtype=tdt) for _ in range(4))
    scale = float(np.float32(1.0 / math.sqrt(D)))
    o, lse = ea.fwd(q, k, v, scale=scale, causal=causal)
    dq, dk, dv, delta = ea.bwd(q, k, v, o, lse, do, scale=scale, causal=causal)
    torch.cuda.synchronize()
    first_past = (1 << 32) // head_bytes
    heads = [0, first_past - 1, first_past, H // 2, H - 1]

    def words_of(t):
        return t[:, heads].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    qw, kw, vw, dow = (words_of(t) for t in (q, k, v, do))
    o_ref, lse_ref = oracle_mod.attn_fwd(qw, kw, vw, dtype, scale, causal)
    eo, el = errors(o_to_f64(o[:, heads]), lse[:, heads].cpu().numpy().astype(np.float64), o_ref, lse_ref)
    assert eo <= TOL_O[dtype], f"max|dO| {eo:.3e}"
    assert el <= TOL_LSE, f"max dLSE {el:.3e}"
    ref = oracle_mod.attn_bwd(qw, kw, vw, dow, dtype, scale, causal)
    tol = 4 * U[dtype]
    for name, t, r in zip(("dq", "dk", "dv", "delta"), (dq, dk, dv, delta), ref):
        x = t[:, heads].float().cpu().numpy().astype(np.float64)
        assert np.abs(x - r).max() <= tol * max(1.0, np.abs(r).max()), name
    del q, k, v, do, o, lse, dq, dk, dv, delta
    torch.cuda.empty_cache()
