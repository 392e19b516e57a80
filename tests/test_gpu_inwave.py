"""GPU parity of the D=256 in-wave pipelined kernel, which runs the D=256
forward where the grid holds at least 512 query tiles of 128 rows (smaller
grids take the 64-row kernel that the other D=256 tests reach).

Same bars as test_gpu_parity (every output element against the fp64
oracle), plus the race canary of test_gpu_variants for this shape: kernel 1
with the same tile shape and one or two stages must give the same bits.
"""

import numpy as np
import pytest

from exact_attention_52_amd import inputs

from gpu_util import TOL_LSE, TOL_O, errors, o_to_f64, scale_for, to_dev
from test_gpu_parity import check_full
from test_gpu_strided import check

pytestmark = pytest.mark.gpu

# 3 * 57 heads of 300 query rows: 513 tiles of 128 rows, the last of each
# head ragged (44 rows)
B, H, S = 3, 57, 300


@pytest.fixture(scope="module")
def ea():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_52_amd as m
    m._lib.load()
    return m


def test_shape_selects_the_inwave_kernel(ea):
    assert ea.attn_fwd_plan(B, H, S, 256, True, 1)["block_m"] == 128
    assert ea.attn_fwd_plan(4, 16, 1037, 256, True, 1)["block_m"] == 128
    assert ea.attn_fwd_plan(2, 3, 1037, 256, True, 1)["block_m"] == 64


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("mult", [1.0, 2.0])
def test_inwave_parity(ea, oracle_mod, dtype, causal, mult):
    # mult 2: peaky scores, so rows rescale their running max on later tiles
    check_full(ea, oracle_mod, B, H, S, 256, dtype, causal, seed=11 + int(mult), mult=mult)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Skv", [1, 130, 517])
def test_inwave_unequal_lengths(ea, oracle_mod, dtype, causal, Skv):
    # causal with Skv < Sq leaves the first Sq - Skv queries without keys
    check(ea, oracle_mod, B, H, S, Skv, 256, dtype, causal, seed=Skv + 3)


@pytest.mark.parametrize("causal", [False, True])
def test_inwave_strided_layout(ea, oracle_mod, causal):
    check(ea, oracle_mod, B, H, S, 333, 256, "bf16", causal, seed=5, layout="bshd", out_layout="padded", mult=2.0)


def test_inwave_negative_scale(ea, oracle_mod):
    check_full(ea, oracle_mod, B, H, S, 256, "fp16", True, seed=4, scale=-0.07)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_inwave_race_canary(ea, oracle_mod, dtype, causal):
    # the in-wave kernel overlaps one tile's softmax with the next tile's
    # scores and the previous tile's PV; kernel 1 with its tile shape runs
    # the same per-wave arithmetic step after step (variant 5: one stage,
    # 6: two stages), so any difference in the bits is a schedule bug
    import torch
    b, h, s = 4, 16, 1037
    q, k, v = inputs.gen_qkv(b, h, s, 256, dtype, seed=71, qk_mult=2.0)
    scale = scale_for(256)
    dev = [to_dev(x, dtype) for x in (q, k, v)]
    print(f"inwave canary {dtype} causal={causal}", flush=True)
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
