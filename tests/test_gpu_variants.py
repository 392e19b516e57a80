"""GPU parity of the copy-schedule variants (attn_fwd_variant): every variant
against the fp64 oracle at the forward tolerances; variants 1-4 (one tile
shape per head dim, different copy schedules) bit-identical to each other;
and the race canary: the shipped tile shape of every head dim, run under
other copy schedules (variants 5 and 6, and 1-4 at D=64), bit-identical to
the shipped kernel."""
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
    for var in range(7):
        print(f"variant {var} D={D} {dtype} causal={causal} S={S}", flush=True)
        o, lse = ea.fwd_variant(*dev, var, scale=scale, causal=causal)
        torch.cuda.synchronize()
        eo, el = errors(o_to_f64(o), lse.cpu().numpy().astype(np.float64), o_ref, lse_ref)
        assert eo <= TOL_O[dtype], f"variant {var}: max|dO| {eo:.3e}"
        assert el <= TOL_LSE, f"variant {var}: max dLSE {el:.3e}"
        outs.append((o, lse))
    for var in range(2, 5):
        assert torch.equal(outs[var][0], outs[1][0]) and torch.equal(outs[var][1], outs[1][1]), var
    same_as_shipped = (1, 2, 3, 4, 5, 6) if D == 64 else (5, 6)
    for var in same_as_shipped:
        assert torch.equal(outs[var][0], outs[0][0]) and torch.equal(outs[var][1], outs[0][1]), var


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("S", [300, 1037])
def test_shipped_schedules_race_canary(ea, oracle_mod, D, dtype, causal, S):
    # The shipped kernels overlap copies, barriers and (D=128) two wave
    # groups' phases; variant 5 runs the same tile shape one step after
    # another with a single LDS stage.  Same per-wave arithmetic, so any
    # difference in the bits is a schedule bug (a read of a stage before its
    # copy landed, or a copy over a stage still being read).
    import torch
    q, k, v = inputs.gen_qkv(2, 3, S, D, dtype, seed=7 * S + D, qk_mult=2.0)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    dev = [to_dev(x, dtype) for x in (q, k, v)]
    print(f"canary D={D} {dtype} causal={causal} S={S}", flush=True)
    o0, l0 = ea.fwd_variant(*dev, 0, scale=scale, causal=causal)
    o5, l5 = ea.fwd_variant(*dev, 5, scale=scale, causal=causal)
    o6, l6 = ea.fwd_variant(*dev, 6, scale=scale, causal=causal)
    o1, l1 = ea.fwd(*dev, scale=scale, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    assert torch.equal(o5, o0) and torch.equal(l5, l0)
    assert torch.equal(o6, o0) and torch.equal(l6, l0)
    o_ref, lse_ref = oracle_mod.attn_fwd(q, k, v, dtype, scale, causal)
    eo, el = errors(o_to_f64(o0), l0.cpu().numpy().astype(np.float64), o_ref, lse_ref)
    assert eo <= TOL_O[dtype] and el <= TOL_LSE, (eo, el)
