"""GPU parity of attn_fwd_strided: queries and keys of different lengths and
strided layouts, against the fp64 oracle (which works on contiguous arrays).

Causal keeps key j for query i iff j <= i + Skv - Sq; a query with no key
gets O = 0 and LSE = -inf exactly.
"""
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


def gen(B, H, Sq, Skv, D, dtype, seed, mult=1.0):
    q, _, _ = inputs.gen_qkv(B, H, Sq, D, dtype, seed=seed, qk_mult=mult)
    _, k, v = inputs.gen_qkv(B, H, Skv, D, dtype, seed=seed + 1, qk_mult=mult)
    return q, k, v


def as_layout(t, layout):
    """The same [B,H,S,D] values in another memory layout (a strided view)."""
    import torch
    B, H, S, D = t.shape
    if layout == "bhsd":
        return t
    if layout == "bshd":  # rows of a head H*D apart, heads D apart
        return t.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    if layout == "padded":  # 8 spare elements after every row
        buf = torch.zeros((B, H, S, D + 8), dtype=t.dtype, device=t.device)
        buf[..., :D] = t
        return buf[..., :D]
    raise ValueError(layout)


def empty_out(B, H, Sq, D, dtype, layout):
    import torch
    from gpu_util import torch_dtype
    o = torch.full((B, H, Sq, D), float("nan"), dtype=torch_dtype(dtype), device="cuda:0")
    return as_layout(o, layout)


def check(ea, oracle_mod, B, H, Sq, Skv, D, dtype, causal, seed, layout="bhsd", out_layout="bhsd",
          mult=1.0):
    import torch
    q, k, v = gen(B, H, Sq, Skv, D, dtype, seed, mult)
    scale = scale_for(D)
    print(f"case B={B} H={H} Sq={Sq} Skv={Skv} D={D} {dtype} causal={causal} layout={layout}/{out_layout}",
          flush=True)
    dq, dk, dv = (as_layout(to_dev(x, dtype), layout) for x in (q, k, v))
    out = empty_out(B, H, Sq, D, dtype, out_layout)
    o, lse = ea.fwd(dq, dk, dv, scale=scale, causal=causal, out=out)
    torch.cuda.synchronize()
    o, lse = o_to_f64(o), lse.cpu().numpy().astype(np.float64)
    o_ref, lse_ref = oracle_mod.attn_fwd(q, k, v, dtype, scale, causal)
    empty = np.isneginf(lse_ref)
    assert np.all(o[empty] == 0.0) and np.all(np.isneginf(lse[empty]))
    live = ~empty
    assert np.all(np.isfinite(o[live])) and np.all(np.isfinite(lse[live]))
    eo, el = errors(o[live], lse[live], o_ref[live], lse_ref[live])
    assert eo <= TOL_O[dtype], f"max|dO| {eo:.3e}"
    assert el <= TOL_LSE, f"max dLSE {el:.3e}"
    return o, lse


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Sq,Skv", [(1, 300), (17, 513), (200, 64), (300, 17), (64, 1), (513, 200)])
def test_unequal_lengths(ea, oracle_mod, D, dtype, causal, Sq, Skv):
    check(ea, oracle_mod, 2, 2, Sq, Skv, D, dtype, causal, seed=Sq * 7 + Skv + D)


@pytest.mark.parametrize("D,dtype", [(64, "fp16"), (128, "bf16"), (128, "fp16"), (256, "bf16")])
@pytest.mark.parametrize("layout,out_layout", [("bshd", "bshd"), ("padded", "bhsd"), ("bhsd", "padded")])
@pytest.mark.parametrize("causal", [False, True])
def test_strided_layouts(ea, oracle_mod, D, dtype, layout, out_layout, causal):
    check(ea, oracle_mod, 2, 3, 130, 257, D, dtype, causal, seed=D + 5, layout=layout,
          out_layout=out_layout, mult=2.0)


@pytest.mark.parametrize("D", [64, 128, 256])
def test_no_keys_at_all(ea, D):
    import torch
    from gpu_util import torch_dtype
    q = torch.randn(1, 2, 40, D, device="cuda:0").to(torch_dtype("bf16"))
    k = torch.empty(1, 2, 0, D, device="cuda:0", dtype=q.dtype)
    for causal in (False, True):
        o, lse = ea.fwd(q, k, k, causal=causal, out=torch.full_like(q, float("nan")))
        torch.cuda.synchronize()
        assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


@pytest.mark.parametrize("D,dtype,causal", [(64, "fp16", True), (128, "fp16", False), (128, "bf16", True),
                                            (256, "bf16", True)])
def test_strided_equals_plain_bitwise(ea, D, dtype, causal):
    # the layout changes the addresses, not the arithmetic
    import torch
    q, k, v = gen(2, 4, 333, 333, D, dtype, seed=D)
    dq, dk, dv = (to_dev(x, dtype) for x in (q, k, v))
    o1, l1 = ea.fwd(dq, dk, dv, causal=causal)
    o2, l2 = ea.fwd(*(as_layout(x, "bshd") for x in (dq, dk, dv)), causal=causal,
                    out=empty_out(2, 4, 333, D, dtype, "padded"))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
