"""attn_bwd_noalloc through the C ABI: the backward with D_i in the library's
own device scratch (no allocation, no delta argument) against attn_bwd on the
same inputs, bit for bit (same kernels), and against the fp64 oracle's
backward at the backward tolerance (4u times the tensor's maximum).  Two
calls in a row, the second on a smaller problem, so the second reuses the
scratch the first left behind."""
import math

import numpy as np
import pytest

from exact_attention_52_amd import inputs

from gpu_util import to_dev

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


def rel_err(x, ref):
    if ref.size == 0:
        return 0.0
    return float(np.abs(x - ref).max() / max(1.0, np.abs(ref).max()))


def check_call(ea, oracle_mod, B, H, Sq, Skv, D, dtype, causal, seed):
    import torch
    print(f"noalloc bwd B={B} H={H} Sq={Sq} Skv={Skv} D={D} {dtype} causal={causal}", flush=True)
    q, _, _ = inputs.gen_qkv(B, H, Sq, D, dtype, seed=seed)
    _, k, v = inputs.gen_qkv(B, H, Skv, D, dtype, seed=seed + 1)
    do, _, _ = inputs.gen_qkv(B, H, Sq, D, dtype, seed=seed + 2)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    tq, tk, tv, tdo = (to_dev(x, dtype) for x in (q, k, v, do))
    o, lse = ea.fwd(tq, tk, tv, scale=scale, causal=causal)
    ref_dq, ref_dk, ref_dv, _ = ea.bwd(tq, tk, tv, o, lse, tdo, scale=scale, causal=causal)
    dq = torch.full_like(tq, float("nan"))
    dk = torch.full_like(tk, float("nan"))
    dv = torch.full_like(tv, float("nan"))
    dt = 0 if dtype == "fp16" else 1
    st = ea._lib.attn_bwd_noalloc(tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                  tdo.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, Sq, Skv, D,
                                  scale, causal, dt, torch.cuda.current_stream().cuda_stream)
    assert st == 0, ea._lib.last_error()
    torch.cuda.synchronize()
    assert torch.equal(dq, ref_dq) and torch.equal(dk, ref_dk) and torch.equal(dv, ref_dv)
    ref = oracle_mod.attn_bwd(q, k, v, do, dtype, scale, causal)
    got = [t.float().cpu().numpy().astype(np.float64) for t in (dq, dk, dv)]
    for name, g, r in zip(("dq", "dk", "dv"), got, ref[:3]):
        e = rel_err(g, r)
        print(f"  {name}: rel err {e:.2e} (tol {4 * U[dtype]:.2e})", flush=True)
        assert e <= 4 * U[dtype], name


def test_noalloc_matches_attn_bwd_on_two_calls_second_smaller(ea, oracle_mod):
    check_call(ea, oracle_mod, 2, 3, 700, 700, 128, "fp16", True, seed=41)
    check_call(ea, oracle_mod, 1, 2, 150, 333, 64, "bf16", False, seed=42)


def test_noalloc_every_head_dim(ea, oracle_mod):
    check_call(ea, oracle_mod, 1, 2, 260, 260, 256, "bf16", True, seed=43)
    check_call(ea, oracle_mod, 1, 1, 97, 97, 64, "fp16", True, seed=44)
