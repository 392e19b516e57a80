"""GPU parity: the gfx950 kernels through the C ABI against the fp64 oracle.

Bar: max |O_gpu - O_ref| <= 2e-3 (fp16) / 1.6e-2 (bf16) over every output
element, and |LSE_gpu - LSE_ref| <= 1e-4 * max(1, |LSE_ref|).
"""
import math

import numpy as np
import pytest

from exact_attention_52_amd import inputs

from gpu_util import TOL_LSE, TOL_O, errors, o_to_f64, scale_for, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ea():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_52_amd as m
    m._lib.load()
    return m


def run(ea, q, k, v, dtype, scale, causal):
    import torch
    o, lse = ea.fwd(to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), scale=scale, causal=causal)
    torch.cuda.synchronize()
    return o_to_f64(o), lse.cpu().numpy().astype(np.float64)


def check_full(ea, oracle_mod, B, H, S, D, dtype, causal, seed=0, mult=1.0, scale=None):
    q, k, v = inputs.gen_qkv(B, H, S, D, dtype, seed=seed, qk_mult=mult)
    scale = scale_for(D) if scale is None else scale
    print(f"case B={B} H={H} S={S} D={D} {dtype} causal={causal} seed={seed} mult={mult}", flush=True)
    o, lse = run(ea, q, k, v, dtype, scale, causal)
    o_ref, lse_ref = oracle_mod.attn_fwd(q, k, v, dtype, scale, causal)
    eo, el = errors(o, lse, o_ref, lse_ref)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    assert eo <= TOL_O[dtype], f"max|dO| {eo:.3e}"
    assert el <= TOL_LSE, f"max dLSE {el:.3e}"
    return q, k, v, o, lse


# --------------------------------------------------------------------------
# small shapes, whole outputs compared: several tiles plus a ragged tail
# --------------------------------------------------------------------------
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("S", [1, 17, 64, 200, 300, 513])
def test_parity_small(ea, oracle_mod, D, dtype, causal, S):
    check_full(ea, oracle_mod, 2, 2, S, D, dtype, causal, seed=S + D)


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_parity_peaky_inputs(ea, oracle_mod, D, dtype):
    # Q, K ~ 2 N(0,1): the running max keeps moving, rescaling O often
    check_full(ea, oracle_mod, 1, 3, 777, D, dtype, False, seed=5, mult=2.0)
    check_full(ea, oracle_mod, 1, 3, 777, D, dtype, True, seed=6, mult=2.0)


def test_parity_c1_whole(ea, oracle_mod):
    B, H, S, D, dtype, causal, mult = inputs.WORKLOADS["c1_b1h2s128d64_fp16"]
    check_full(ea, oracle_mod, B, H, S, D, dtype, causal, seed=0, mult=mult)


# --------------------------------------------------------------------------
# the five workloads at full size: every O and LSE element against the oracle
# --------------------------------------------------------------------------
@pytest.mark.parametrize("name", list(inputs.WORKLOADS))
def test_parity_workload_full(ea, oracle_mod, name):
    B, H, S, D, dtype, causal, mult = inputs.WORKLOADS[name]
    print(f"workload {name}", flush=True)
    q, k, v = inputs.gen_qkv(B, H, S, D, dtype, seed=0, qk_mult=mult)
    scale = scale_for(D)
    o, lse = run(ea, q, k, v, dtype, scale, causal)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    o_ref, lse_ref = oracle_mod.attn_fwd(q, k, v, dtype, scale, causal)
    eo, el = errors(o, lse, o_ref, lse_ref)
    print(f"  all {B * H * S} rows, {o.size} O elements: max|dO|={eo:.3e} max dLSE={el:.3e}", flush=True)
    assert eo <= TOL_O[dtype], f"max|dO| {eo:.3e}"
    assert el <= TOL_LSE, f"max dLSE {el:.3e}"
    if causal:
        # causal row 0 attends to key 0 only: O_0 is V_0 exactly
        vv = v.reshape(B * H, S, D)[:, 0]
        assert np.array_equal(o.reshape(B * H, S, D)[:, 0], inputs.bits_to_float(vv, dtype).astype(np.float64))


# --------------------------------------------------------------------------
# properties
# --------------------------------------------------------------------------
@pytest.mark.parametrize("D,dtype", [(64, "fp16"), (128, "bf16"), (256, "bf16")])
def test_deterministic_and_slice_independent(ea, D, dtype):
    import torch
    B, H, S = 2, 3, 700
    q, k, v = inputs.gen_qkv(B, H, S, D, dtype, seed=21)
    dq, dk, dv = (to_dev(x, dtype) for x in (q, k, v))
    o1, l1 = ea.fwd(dq, dk, dv, causal=True)
    o2, l2 = ea.fwd(dq, dk, dv, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # one (b, h) run alone gives the same bits as inside the batch
    b, h = 1, 2
    os_, ls_ = ea.fwd(dq[b:b + 1, h:h + 1].contiguous(), dk[b:b + 1, h:h + 1].contiguous(),
                      dv[b:b + 1, h:h + 1].contiguous(), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(os_[0, 0], o1[b, h]) and torch.equal(ls_[0, 0], l1[b, h])


@pytest.mark.parametrize("D,dtype", [(64, "fp16"), (128, "fp16"), (256, "bf16")])
@pytest.mark.parametrize("causal", [False, True])
def test_zero_query_closed_form(ea, D, dtype, causal):
    B, H, S = 1, 2, 333
    _, k, v = inputs.gen_qkv(B, H, S, D, dtype, seed=22)
    q = np.zeros_like(k)
    o, lse = run(ea, q, k, v, dtype, 0.5, causal)
    vv = inputs.bits_to_float(v, dtype).astype(np.float64)
    n = np.arange(1, S + 1) if causal else np.full(S, S)
    ref = np.cumsum(vv, axis=2) / n[:, None] if causal else np.broadcast_to(vv.mean(axis=2, keepdims=True), vv.shape)
    assert np.abs(o - ref).max() <= TOL_O[dtype]
    assert np.abs(lse - np.log(n)).max() <= TOL_LSE * max(1.0, math.log(S))


@pytest.mark.parametrize("D,dtype", [(64, "fp16"), (128, "fp16"), (256, "bf16")])
def test_rising_max_every_tile(ea, oracle_mod, D, dtype):
    # every later key scores higher than all earlier ones: the running max
    # rises in every key tile, so every tile rescales O
    B, H, S = 1, 1, 640
    qf = np.zeros((B, H, S, D))
    qf[..., 0] = 1.0
    kf = np.zeros((B, H, S, D))
    kf[..., 0] = np.arange(S) / 16.0
    q, k = inputs.round_to_bits(qf, dtype), inputs.round_to_bits(kf, dtype)
    _, _, v = inputs.gen_qkv(B, H, S, D, dtype, seed=23)
    for causal in (False, True):
        o, lse = run(ea, q, k, v, dtype, 1.0, causal)
        o_ref, lse_ref = oracle_mod.attn_fwd(q, k, v, dtype, 1.0, causal)
        eo, el = errors(o, lse, o_ref, lse_ref)
        assert eo <= TOL_O[dtype] and el <= TOL_LSE, (causal, eo, el)


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("step", [3.0, 6.0])
def test_rising_max_in_steps(ea, oracle_mod, D, dtype, step):
    # the scores of keys 64m .. 64m+63 are step * m: the row max rises by
    # step * log2(e) (4.3 or 8.7) per 64 keys, below or just above the 2^8
    # slack of the lagging reference max, so rescales fire on some key tiles
    # and not on others, and P runs up towards 2^8 between them
    B, H, S = 1, 2, 700
    qf = np.zeros((B, H, S, D))
    qf[..., 0] = 1.0
    kf = np.zeros((B, H, S, D))
    kf[..., 0] = step * (np.arange(S) // 64)
    q, k = inputs.round_to_bits(qf, dtype), inputs.round_to_bits(kf, dtype)
    _, _, v = inputs.gen_qkv(B, H, S, D, dtype, seed=29)
    for causal in (False, True):
        o, lse = run(ea, q, k, v, dtype, 1.0, causal)
        o_ref, lse_ref = oracle_mod.attn_fwd(q, k, v, dtype, 1.0, causal)
        eo, el = errors(o, lse, o_ref, lse_ref)
        assert eo <= TOL_O[dtype] and el <= TOL_LSE, (causal, eo, el)


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_negative_scale(ea, oracle_mod, D, dtype, causal):
    # the page's sm_scale is a plain f32: a negative scale flips the softmax
    # towards the least similar keys; the kernels apply it as -Q times |scale|
    check_full(ea, oracle_mod, 1, 2, 333, D, dtype, causal, seed=D + 31, mult=2.0, scale=-float(scale_for(D)))


def test_scale_zero_is_uniform(ea):
    B, H, S, D = 1, 2, 150, 128
    q, k, v = inputs.gen_qkv(B, H, S, D, "fp16", seed=24)
    o, lse = run(ea, q, k, v, "fp16", 0.0, False)
    vv = inputs.bits_to_float(v, "fp16").astype(np.float64)
    assert np.abs(o - vv.mean(axis=2, keepdims=True)).max() <= TOL_O["fp16"]
    assert np.abs(lse - math.log(S)).max() <= TOL_LSE * math.log(S)


def test_side_stream_and_preallocated_outputs(ea, oracle_mod):
    import torch
    B, H, S, D = 1, 2, 260, 64
    q, k, v = inputs.gen_qkv(B, H, S, D, "bf16", seed=25)
    dq, dk, dv = (to_dev(x, "bf16") for x in (q, k, v))
    out = torch.full_like(dq, float("nan"))
    lse = torch.full((B, H, S), float("nan"), device="cuda:0")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ea.fwd(dq, dk, dv, scale=0.125, causal=True, out=out, lse=lse)
    s.synchronize()
    o_ref, lse_ref = oracle_mod.attn_fwd(q, k, v, "bf16", 0.125, True)
    eo, el = errors(o_to_f64(out), lse.cpu().numpy().astype(np.float64), o_ref, lse_ref)
    assert eo <= TOL_O["bf16"] and el <= TOL_LSE


def test_empty_and_invalid_through_binding(ea):
    import torch
    z = torch.empty((0, 2, 16, 64), dtype=torch.float16, device="cuda:0")
    o, lse = ea.fwd(z, z, z)
    assert o.shape == z.shape and lse.shape == (0, 2, 16)
    x = torch.zeros((1, 1, 16, 96), dtype=torch.float16, device="cuda:0")
    with pytest.raises(ea.AttnError) as e:
        ea.fwd(x, x, x)
    assert e.value.status == 3
