"""GPU parity of the unfused comparator (attn_fwd_unfused) against the fp64
oracle, with the forward's tolerances: its P is rounded to the input dtype
before P V, as the fused kernels round theirs."""
import math

import numpy as np
import pytest

from exact_attention_52_amd import inputs

from gpu_util import TOL_LSE, TOL_O, errors, o_to_f64, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ea():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_52_amd as m
    m._lib.load()
    return m


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("S", [1, 77, 300, 1025, 8200])
def test_unfused_parity(ea, oracle_mod, D, dtype, causal, S):
    import torch
    B, H = (1, 1) if S > 4096 else (2, 2)
    print(f"unfused case B={B} H={H} S={S} D={D} {dtype} causal={causal}", flush=True)
    q, k, v = inputs.gen_qkv(B, H, S, D, dtype, seed=S + D, qk_mult=2.0 if S == 300 else 1.0)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    o, lse = ea.fwd_unfused(*(to_dev(x, dtype) for x in (q, k, v)), scale=scale, causal=causal)
    torch.cuda.synchronize()
    rows = None if S <= 1025 else np.random.default_rng(S).integers(0, B * H * S, 300)
    o_ref, lse_ref = oracle_mod.attn_fwd(q, k, v, dtype, scale, causal, rows=rows)
    o_g, lse_g = o_to_f64(o), lse.cpu().numpy().astype(np.float64)
    if rows is not None:
        o_g, lse_g = o_g.reshape(-1, D)[rows], lse_g.reshape(-1)[rows]
    eo, el = errors(o_g, lse_g, o_ref, lse_ref)
    assert eo <= TOL_O[dtype], f"max|dO| {eo:.3e}"
    assert el <= TOL_LSE, f"max dLSE {el:.3e}"


def test_unfused_peaky_workload_every_element(ea, oracle_mod):
    # the peaky fp16 workload B=2 H=16 S=4096 D=128 has elements with |O| ~ 4.5,
    # where O's own fp16 rounding leaves under 5e-5 of the 2e-3 bound: every
    # element of O and LSE against the oracle
    import torch
    B, H, S, D, dtype, causal, mult = inputs.WORKLOADS["c4_b2h16s4096d128_fp16_peaky"]
    print("unfused, B=2 H=16 S=4096 D=128 fp16, every element", flush=True)
    q, k, v = inputs.gen_qkv(B, H, S, D, dtype, seed=0, qk_mult=mult)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    o, lse = ea.fwd_unfused(*(to_dev(x, dtype) for x in (q, k, v)), scale=scale, causal=causal)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle_mod.attn_fwd(q, k, v, dtype, scale, causal)
    eo, el = errors(o_to_f64(o), lse.cpu().numpy().astype(np.float64), o_ref, lse_ref)
    print(f"  max|dO|={eo:.3e} max dLSE={el:.3e}", flush=True)
    assert eo <= TOL_O[dtype], f"max|dO| {eo:.3e}"
    assert el <= TOL_LSE, f"max dLSE {el:.3e}"
    torch.cuda.empty_cache()
