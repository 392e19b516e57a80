"""GPU parity of the copy-schedule variants (attn_fwd_variant): every variant
against the fp64 oracle at the forward tolerances, and variants 1-4 (one tile
shape per head dim, different copy schedules) bit-identical to each other."""
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


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("S", [70, 389])
def test_variants(ea, oracle_mod, D, dtype, causal, S):
    import torch
    q, k, v = inputs.gen_qkv(2, 2, S, D, dtype, seed=S + D, qk_mult=2.0)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    dev = [to_dev(x, dtype) for x in (q, k, v)]
    o_ref, lse_ref = oracle_mod.attn_fwd(q, k, v, dtype, scale, causal)
    outs = []
    for var in range(5):
        print(f"variant {var} D={D} {dtype} causal={causal} S={S}", flush=True)
        o, lse = ea.fwd_variant(*dev, var, scale=scale, causal=causal)
        torch.cuda.synchronize()
        eo, el = errors(o_to_f64(o), lse.cpu().numpy().astype(np.float64), o_ref, lse_ref)
        assert eo <= TOL_O[dtype], f"variant {var}: max|dO| {eo:.3e}"
        assert el <= TOL_LSE, f"variant {var}: max dLSE {el:.3e}"
        outs.append((o, lse))
    for var in range(2, 5):
        assert torch.equal(outs[var][0], outs[1][0]) and torch.equal(outs[var][1], outs[1][1]), var
