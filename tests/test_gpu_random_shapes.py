"""Forward and backward on seeded random shapes against the fp64 oracle.

Each case draws B, H, Sq, Skv, D, dtype, causal, the score spread (Q and K
scaled by 1 or 2, the larger making peaky rows), the sign of the scale and
the memory layout (contiguous, [B,S,H,D] views, padded rows) from a fixed
seed, so that the combinations the hand-picked cases leave out (ragged query
and key tails in every kernel, Sq much larger or smaller than Skv with the
causal offset, tiles that are both diagonal and ragged) are exercised too.
Every output element is compared: O within the forward tolerance, LSE within
1e-4 * max(1, |LSE|), the gradients within 4u of each tensor's largest
element (the backward's bound, see test_gpu_bwd.py).
"""
import math

import numpy as np
import pytest

from exact_attention_52_amd import inputs

from gpu_util import TOL_LSE, TOL_O, errors, o_to_f64, to_dev

pytestmark = pytest.mark.gpu

U = {"fp16": 2.0 ** -11, "bf16": 2.0 ** -8}
N_CASES = 40


@pytest.fixture(scope="module")
def ea():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_52_amd as m
    m._lib.load()
    return m


def draw(i):
    r = np.random.default_rng(1000 + i)
    D = int(r.choice([64, 128, 256]))
    return dict(B=int(r.integers(1, 3)), H=int(r.integers(1, 4)), Sq=int(r.integers(1, 600)),
                Skv=int(r.integers(1, 600)), D=D, dtype=str(r.choice(["fp16", "bf16"])),
                causal=bool(r.integers(0, 2)), mult=float(r.choice([1.0, 2.0])),
                sign=float(r.choice([1.0, -1.0])), layout=str(r.choice(["bhsd", "bshd", "padded"])))


def as_layout(t, layout):
    import torch
    B, H, S, D = t.shape
    if layout == "bhsd":
        return t
    if layout == "bshd":
        return t.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    buf = torch.zeros((B, H, S, D + 8), dtype=t.dtype, device=t.device)
    buf[..., :D] = t
    return buf[..., :D]


def rel_err(x, ref):
    if ref.size == 0:
        return 0.0
    return float(np.abs(x - ref).max() / max(1.0, np.abs(ref).max()))


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape(ea, oracle_mod, i):
    import torch
    c = draw(i)
    B, H, Sq, Skv, D, dtype = c["B"], c["H"], c["Sq"], c["Skv"], c["D"], c["dtype"]
    print(f"random case {i}: {c}", flush=True)
    q, _, _ = inputs.gen_qkv(B, H, Sq, D, dtype, seed=2 * i, qk_mult=c["mult"])
    _, k, v = inputs.gen_qkv(B, H, Skv, D, dtype, seed=2 * i + 1, qk_mult=c["mult"])
    do, _, _ = inputs.gen_qkv(B, H, Sq, D, dtype, seed=7000 + i)
    scale = c["sign"] * float(np.float32(1.0 / math.sqrt(D)))
    dev = [as_layout(to_dev(x, dtype), c["layout"]) for x in (q, k, v, do)]
    o, lse = ea.fwd(*dev[:3], scale=scale, causal=c["causal"])
    dq, dk, dv, delta = ea.bwd(*dev[:3], o, lse, dev[3], scale=scale, causal=c["causal"])
    torch.cuda.synchronize()

    o_ref, lse_ref = oracle_mod.attn_fwd(q, k, v, dtype, scale, c["causal"])
    og, lg = o_to_f64(o), lse.cpu().numpy().astype(np.float64)
    finite = np.isfinite(lse_ref)  # rows with no key: LSE = -inf on both sides
    assert np.array_equal(np.isfinite(lg), finite), "rows without keys differ"
    assert np.all(og[~finite] == 0.0), "O of a row without keys is not 0"
    eo, el = errors(og[finite], lg[finite], o_ref[finite], lse_ref[finite])
    assert eo <= TOL_O[dtype], f"max|dO| {eo:.3e}"
    assert el <= TOL_LSE, f"max dLSE {el:.3e}"

    ref = oracle_mod.attn_bwd(q, k, v, do, dtype, scale, c["causal"])
    tol = 4 * U[dtype]
    for name, t, r in zip(("dq", "dk", "dv", "delta"), (dq, dk, dv, delta), ref):
        x = t.float().cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(x)), f"{name} not finite"
        e = rel_err(x, r)
        assert e <= tol, f"{name}: {e:.3e} > {tol:.3e}"
