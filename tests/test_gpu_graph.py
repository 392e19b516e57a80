"""attn_fwd and attn_bwd captured in a HIP graph.

Both calls only enqueue kernels on the caller's stream (no allocation, no
memset, no synchronisation), so a graph captured from them replays the same
work on whatever the captured buffers hold at replay time.  Each case
captures forward + backward once, then replays the graph three times with
eager work and synchronisations in between (new inputs copied into the
captured buffers, every output overwritten with NaN), and every replay must
equal, bit for bit, an eager run on the same inputs.
"""
import math

import numpy as np
import pytest

from exact_attention_52_amd import inputs

from gpu_util import to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ea():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_52_amd as m
    m._lib.load()
    return m


def eager(ea, q, k, v, do, scale, causal):
    o, lse = ea.fwd(q, k, v, scale=scale, causal=causal)
    dq, dk, dv, delta = ea.bwd(q, k, v, o, lse, do, scale=scale, causal=causal)
    return o, lse, dq, dk, dv, delta


# (B, H, S, D): small shapes with a ragged tail for each head dim, and one
# D=256 grid large enough for the in-wave kernel
@pytest.mark.parametrize("B,H,S,D", [(2, 3, 300, 64), (2, 3, 300, 128), (2, 3, 300, 256), (4, 16, 1024, 256)])
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_graph_replays_equal_eager(ea, B, H, S, D, dtype, causal):
    import torch
    print(f"graph case B={B} H={H} S={S} D={D} {dtype} causal={causal}", flush=True)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    sets = []
    for seed in (11, 12):
        q, k, v = inputs.gen_qkv(B, H, S, D, dtype, seed=seed)
        do, _, _ = inputs.gen_qkv(B, H, S, D, dtype, seed=seed + 100)
        sets.append(tuple(to_dev(x, dtype) for x in (q, k, v, do)))
    refs = [eager(ea, *s, scale, causal) for s in sets]
    torch.cuda.synchronize()

    # the captured buffers
    q, k, v, do = (x.clone() for x in sets[0])
    o = torch.empty_like(q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty_like(lse)
    outs = (o, lse, dq, dk, dv, delta)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ea.fwd(q, k, v, scale=scale, causal=causal, out=o, lse=lse)
        ea.bwd(q, k, v, o, lse, do, scale=scale, causal=causal, dq=dq, dk=dk, dv=dv, delta=delta)
    torch.cuda.synchronize()

    for r, which in enumerate((0, 1, 0)):
        for dst, src in zip((q, k, v, do), sets[which]):
            dst.copy_(src)
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("o", "lse", "dq", "dk", "dv", "delta"), outs, refs[which]):
            assert torch.equal(got, want), f"replay {r} (input set {which}): {name} differs from the eager run"
    del g
