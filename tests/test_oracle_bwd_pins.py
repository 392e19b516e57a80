"""Pins of the oracle's attention backward (CPU only).

The backward is pinned to facts other than its own formulas:
  * it is the derivative of the forward: central finite differences of the
    float64 forward (itself tied to the pinned 16-bit forward) for every
    input element on small problems, causal and not, Sq < Skv and Sq > Skv;
  * torch's float64 autograd through a plain softmax attention;
  * exact consequences of the softmax Jacobian: every row of dS sums to 0, so
    the dK rows of a head sum to 0; the dV rows sum to the dO rows that see a
    key; sum_i q_i.dQ_i = sum_j k_j.dK_j (both are sum dS_ij s_ij);
  * D_i = rowsum(dP * P) equals dO_i . O_i (the page names both forms);
  * closed forms: dO = 0; equal V rows; one key; scale 0; rows with no key.
"""
import numpy as np
import pytest

import oracle


def rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def problem(B, H, Sq, Skv, D, seed):
    return (rand((B, H, Sq, D), seed), rand((B, H, Skv, D), seed + 1), rand((B, H, Skv, D), seed + 2),
            rand((B, H, Sq, D), seed + 3))


CASES = [(1, 2, 5, 5, 4, False), (1, 2, 5, 5, 4, True), (2, 1, 3, 7, 6, True), (1, 1, 6, 4, 3, True),
         (1, 2, 4, 9, 5, False), (1, 1, 7, 3, 2, False)]


def test_fwd_f64_is_the_pinned_16bit_forward():
    from exact_attention_52_amd import inputs
    for dtype in ("fp16", "bf16"):
        for causal in (False, True):
            q, _, _ = inputs.gen_qkv(2, 3, 37, 64, dtype, seed=4)
            _, k, v = inputs.gen_qkv(2, 3, 53, 64, dtype, seed=5)
            o16, l16 = oracle.attn_fwd(q, k, v, dtype, 0.125, causal)
            dec = [oracle.decode(x, dtype) for x in (q, k, v)]
            o64, l64 = oracle.attn_fwd_f64(*dec, 0.125, causal)
            assert np.abs(o64 - o16).max() <= 1e-14
            assert np.abs(l64 - l16).max() <= 1e-13


@pytest.mark.parametrize("scale", [0.7, -0.45])
@pytest.mark.parametrize("B,H,Sq,Skv,D,causal", CASES)
def test_bwd_is_the_derivative_of_the_forward(B, H, Sq, Skv, D, causal, scale):
    q, k, v, do = problem(B, H, Sq, Skv, D, seed=Sq * 10 + Skv)

    def loss(q_, k_, v_):
        o, _ = oracle.attn_fwd_f64(q_, k_, v_, scale, causal)
        return float(np.sum(o * do))

    dq, dk, dv, _ = oracle.attn_bwd_f64(q, k, v, do, scale, causal)
    h = 1e-5
    worst = 0.0
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        xs = [q, k, v]
        x = xs[which]
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            saved = x[idx]
            x[idx] = saved + h
            lp = loss(*xs)
            x[idx] = saved - h
            lm = loss(*xs)
            x[idx] = saved
            fd[idx] = (lp - lm) / (2 * h)
        worst = max(worst, np.abs(fd - grad).max())
    assert worst < 1e-7, worst


def torch_bwd(q, k, v, do, scale, causal):
    import torch
    t = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v)]
    Sq, Skv = q.shape[2], k.shape[2]
    s = torch.matmul(t[0], t[1].transpose(-1, -2).contiguous()) * scale
    if causal:
        i = torch.arange(Sq)[:, None]
        j = torch.arange(Skv)[None, :]
        s = s.masked_fill(j > i + (Skv - Sq), float("-inf"))
    o = torch.matmul(torch.softmax(s, dim=-1), t[2])
    o.backward(torch.tensor(do, dtype=torch.float64))
    return [x.grad.numpy() for x in t]


@pytest.mark.parametrize("Sq,Skv,D,causal", [(33, 33, 64, False), (33, 33, 64, True), (20, 50, 128, True),
                                             (50, 20, 32, False), (64, 64, 256, True)])
def test_bwd_matches_torch_float64_autograd(Sq, Skv, D, causal):
    q, k, v, do = problem(2, 2, Sq, Skv, D, seed=D + Sq)
    scale = 1 / np.sqrt(D)
    ours = oracle.attn_bwd_f64(q, k, v, do, scale, causal)[:3]
    ref = torch_bwd(q, k, v, do, scale, causal)
    for a, b in zip(ours, ref):
        assert np.abs(a - b).max() <= 1e-12 * max(1.0, np.abs(b).max())


@pytest.mark.parametrize("causal", [False, True])
def test_softmax_jacobian_identities(causal):
    B, H, Sq, Skv, D = 2, 3, 24, 40, 16
    q, k, v, do = problem(B, H, Sq, Skv, D, seed=11)
    scale = 0.3
    dq, dk, dv, delta = oracle.attn_bwd_f64(q, k, v, do, scale, causal)
    # every query here sees a key (Sq <= Skv), so each row of dS sums to 0
    assert np.abs(dk.sum(axis=2)).max() <= 1e-12
    assert np.abs(dv.sum(axis=2) - do.sum(axis=2)).max() <= 1e-12
    lhs = np.einsum("bhid,bhid->bh", q, dq)
    rhs = np.einsum("bhjd,bhjd->bh", k, dk)
    assert np.abs(lhs - rhs).max() <= 1e-12
    # D_i = rowsum(dP * P) = dO_i . O_i
    o, _ = oracle.attn_fwd_f64(q, k, v, scale, causal)
    assert np.abs(delta - np.einsum("bhid,bhid->bhi", do, o)).max() <= 1e-12


def test_zero_output_gradient():
    q, k, v, _ = problem(1, 2, 9, 9, 8, seed=3)
    for g in oracle.attn_bwd_f64(q, k, v, np.zeros_like(q), 0.5, True):
        assert np.all(g == 0.0)


@pytest.mark.parametrize("causal", [False, True])
def test_equal_value_rows_give_no_score_gradient(causal):
    q, k, _, do = problem(1, 2, 10, 12, 8, seed=6)
    v = np.broadcast_to(rand((1, 2, 1, 8), 9), (1, 2, 12, 8)).copy()
    dq, dk, dv, _ = oracle.attn_bwd_f64(q, k, v, do, 0.5, causal)
    assert np.abs(dq).max() <= 1e-13 and np.abs(dk).max() <= 1e-13
    assert np.abs(dv.sum(axis=2) - do.sum(axis=2)).max() <= 1e-12


def test_one_key():
    q, k, v, do = problem(1, 2, 6, 1, 8, seed=8)
    dq, dk, dv, delta = oracle.attn_bwd_f64(q, k, v, do, 0.5, False)
    assert np.abs(dq).max() <= 1e-14 and np.abs(dk).max() <= 1e-14
    assert np.abs(dv[:, :, 0] - do.sum(axis=2)).max() <= 1e-13
    assert np.abs(delta - np.einsum("bhid,bhd->bhi", do, v[:, :, 0])).max() <= 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_scale_zero_is_uniform_attention(causal):
    B, H, Sq, Skv, D = 1, 2, 5, 8, 4
    q, k, v, do = problem(B, H, Sq, Skv, D, seed=12)
    dq, dk, dv, _ = oracle.attn_bwd_f64(q, k, v, do, 0.0, causal)
    assert np.all(dq == 0.0) and np.all(dk == 0.0)
    want = np.zeros_like(dv)
    for i in range(Sq):
        n = min(Skv, i + 1 + Skv - Sq) if causal else Skv
        want[:, :, :n] += do[:, :, i:i + 1] / n
    assert np.abs(dv - want).max() <= 1e-14


def test_rows_with_no_key_drop_out():
    # causal, Sq > Skv: the first Sq - Skv queries see no key; the gradients
    # equal those of the square problem made of the remaining queries
    B, H, Sq, Skv, D = 1, 2, 9, 4, 8
    q, k, v, do = problem(B, H, Sq, Skv, D, seed=13)
    dq, dk, dv, delta = oracle.attn_bwd_f64(q, k, v, do, 0.4, True)
    cut = Sq - Skv
    assert np.all(dq[:, :, :cut] == 0.0) and np.all(delta[:, :, :cut] == 0.0)
    dq2, dk2, dv2, delta2 = oracle.attn_bwd_f64(q[:, :, cut:], k, v, do[:, :, cut:], 0.4, True)
    assert np.array_equal(dq[:, :, cut:], dq2) and np.array_equal(delta[:, :, cut:], delta2)
    assert np.abs(dk - dk2).max() <= 1e-15 and np.abs(dv - dv2).max() <= 1e-15


def test_16bit_entry_widens_exactly():
    from exact_attention_52_amd import inputs
    for dtype in ("fp16", "bf16"):
        q, k, v = inputs.gen_qkv(1, 2, 19, 64, dtype, seed=7)
        do, _, _ = inputs.gen_qkv(1, 2, 19, 64, dtype, seed=8)
        a = oracle.attn_bwd(q, k, v, do, dtype, 0.125, True)
        b = oracle.attn_bwd_f64(*(oracle.decode(x, dtype) for x in (q, k, v, do)), 0.125, True)
        for x, y in zip(a, b):
            assert np.array_equal(x, y)


@pytest.mark.parametrize("causal", [False, True])
def test_sampled_rows_equal_the_full_backward(causal):
    from exact_attention_52_amd import inputs
    q, _, _ = inputs.gen_qkv(2, 3, 41, 64, "bf16", seed=3)
    _, k, v = inputs.gen_qkv(2, 3, 29, 64, "bf16", seed=4)
    do, _, _ = inputs.gen_qkv(2, 3, 41, 64, "bf16", seed=5)
    dq, _, _, delta = oracle.attn_bwd(q, k, v, do, "bf16", 0.125, causal)
    rows = np.array([0, 5, 40, 41, 100, 2 * 3 * 41 - 1])
    dq_r, delta_r = oracle.attn_bwd_rows(q, k, v, do, "bf16", 0.125, causal, rows)
    assert np.abs(dq_r - dq.reshape(-1, 64)[rows]).max() <= 1e-13
    assert np.abs(delta_r - delta.reshape(-1)[rows]).max() <= 1e-13


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Sq,Skv", [(41, 29), (29, 41), (33, 33)])
def test_sampled_keys_equal_the_full_backward(causal, Sq, Skv):
    from exact_attention_52_amd import inputs
    q, _, _ = inputs.gen_qkv(2, 2, Sq, 64, "fp16", seed=6)
    _, k, v = inputs.gen_qkv(2, 2, Skv, 64, "fp16", seed=7)
    do, _, _ = inputs.gen_qkv(2, 2, Sq, 64, "fp16", seed=8)
    _, dk, dv, _ = oracle.attn_bwd(q, k, v, do, "fp16", 0.125, causal)
    keys = np.array([0, 7, Skv - 1, Skv, 2 * 2 * Skv - 1])
    dk_s, dv_s = oracle.attn_bwd_keys(q, k, v, do, "fp16", 0.125, causal, keys)
    assert np.abs(dk_s - dk.reshape(-1, 64)[keys]).max() <= 1e-13
    assert np.abs(dv_s - dv.reshape(-1, 64)[keys]).max() <= 1e-13
