"""The C-ABI library on the CPU: it loads, exports every declared symbol, plans
launches like the page's launch_params, maps workgroups bijectively, and
rejects every invalid argument before any HIP call."""
import json
import os
import re

import pytest

import exact_attention_52_amd as ea
from exact_attention_52_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")


def declared_functions(header="attn.h"):
    text = open(os.path.join(ROOT, "include", header)).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


def test_library_loads_and_exports_every_declared_symbol():
    lib = _lib.load()
    names = declared_functions()
    assert names, "no declarations parsed"
    assert set(names) == set(_lib.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.attn_abi_version() == _lib.ABI_VERSION
    # no torch types cross the ABI: the header holds only C types
    for hdr_name in ("attn.h", "attn_unfused.h"):
        hdr = open(os.path.join(ROOT, "include", hdr_name)).read()
        assert "torch" not in hdr.lower().replace("pytorch", "")


def test_unfused_library_loads_and_exports_every_declared_symbol():
    lib = _lib.load_unfused()
    names = declared_functions("attn_unfused.h")
    assert set(names) == set(_lib.UNFUSED_EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def _dynamic_symbols(path):
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True, check=True).stdout
    return {ln.split()[-1] for ln in out.splitlines() if ln.strip()}


def test_exported_symbols_in_dynamic_table():
    syms = _dynamic_symbols(_lib.LIB_PATH)
    for n in declared_functions():
        assert n in syms
    usyms = _dynamic_symbols(_lib.UNFUSED_LIB_PATH)
    for n in declared_functions("attn_unfused.h"):
        assert n in usyms


def test_fused_library_links_no_vendor_blas():
    import subprocess
    out = subprocess.run(["readelf", "-d", _lib.LIB_PATH], capture_output=True, text=True, check=True).stdout
    needed = [ln for ln in out.splitlines() if "NEEDED" in ln]
    assert needed and not any(x in ln for ln in needed for x in ("rocblas", "hipblas", "hipblaslt")), needed


def test_status_strings():
    for code in _lib.STATUS:
        assert _lib.status_string(code) != "unknown status"
    assert _lib.status_string(999) == "unknown status"


def test_launch_geometry_matches_page():
    g = json.load(open(os.path.join(GOLDEN, "launch_geometry.json")))
    bm = g["block_m"]
    for c in g["cases"]:
        # the page's rule with its 128-row tile gives its printed grid
        assert -(-c["seq_len_q"] // bm) == c["grid_x"]
        assert c["batch"] * c["heads"] == c["grid_y"]
        # our plan applies the same rule with its own tile height, and the key
        # length never enters the grid
        for D in (64, 128, 256):
            p = ea.attn_fwd_plan(c["batch"], c["heads"], c["seq_len_q"], D, False, 0)
            assert p["num_q_tiles"] == -(-c["seq_len_q"] // p["block_m"])
            assert p["num_workgroups"] == p["num_q_tiles"] * c["grid_y"]
            if p["block_m"] == bm:
                assert p["num_q_tiles"] == c["grid_x"]


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("S", [1, 63, 64, 65, 300, 1024, 8192])
def test_plan_rules(D, S):
    p = ea.attn_fwd_plan(3, 5, S, D, True, 1)
    bm = p["block_m"]
    assert p["num_q_tiles"] == -(-S // bm)
    assert p["num_workgroups"] == p["num_q_tiles"] * 15
    assert p["threads_per_workgroup"] == 64 * p["waves_q"] * p["waves_k"]
    assert bm == 32 * p["waves_q"]
    assert p["lds_bytes"] <= 160 * 1024
    assert p["kv_stages"] == 2
    if D == 256:
        # 64-row query tiles (the page's D=256 tile), except where the grid of
        # 128-row tiles fills the 256 CUs at least twice: the in-wave kernel
        assert bm == (128 if 15 * -(-S // 128) >= 512 else 64)
        assert p["waves_k"] == (1 if bm == 128 else 2)


@pytest.mark.parametrize("B,H,S,bm", [(1, 8, 8192, 128), (1, 8, 8191, 128), (1, 8, 8064, 64), (1, 16, 4096, 128),
                                      (1, 16, 2048, 64), (2, 8, 1024, 64), (4, 128, 128, 128), (1, 511, 128, 64)])
def test_d256_shape_rule(B, H, S, bm):
    # the boundary of the size rule: B*H*ceil(S/128) >= 512
    p = ea.attn_fwd_plan(B, H, S, 256, True, 1)
    assert p["block_m"] == bm, p
    assert p["num_workgroups"] == B * H * -(-S // bm)


def test_supported_and_rejected_head_dims_and_types():
    g = json.load(open(os.path.join(GOLDEN, "launch_geometry.json")))
    for D in g["supported_head_dims"]:
        ea.attn_fwd_plan(1, 1, 128, D, False, 0)
    for D in g["rejected_head_dims"] + [0, 32, 512, -64]:
        with pytest.raises(_lib.AttnError) as e:
            ea.attn_fwd_plan(1, 1, 128, D, False, 0)
        assert e.value.status == 3 and "head_dim" in e.value.detail
    for dt in (2, -1, 7):
        with pytest.raises(_lib.AttnError) as e:
            ea.attn_fwd_plan(1, 1, 128, 64, False, dt)
        assert e.value.status == 4


@pytest.mark.parametrize("D,causal", [(64, False), (64, True), (128, True), (256, True), (128, False)])
@pytest.mark.parametrize("B,H,S", [(1, 1, 1), (2, 3, 1000), (1, 8, 8192), (3, 1, 257), (4, 16, 2048)])
def test_workgroup_map_is_bijection_and_longest_first(B, H, S, D, causal):
    p = ea.attn_fwd_plan(B, H, S, D, causal, 0)
    G, nq = p["num_workgroups"], p["num_q_tiles"]
    seen = set()
    last = {}
    heads = B * H
    chunk_heads = {}  # XCD -> heads of its current chunk
    for wg in range(G):
        t, bh = ea.attn_fwd_workgroup_tile(B, H, S, D, causal, 0, wg)
        assert 0 <= t < nq and 0 <= bh < B * H
        seen.add((t, bh))
        if causal:
            key = wg % 8
            if heads % 8 == 0:
                assert bh % 8 == wg % 8  # a head's tiles share one XCD
                # each XCD works through chunks of its heads; within a chunk
                # its tiles come in order of non-increasing cost (tile t
                # costs t + 1 key tiles), and a new chunk starts at the last
                # tile of heads the XCD has not seen yet
                cur = chunk_heads.setdefault(key, set())
                if bh not in cur:
                    if last.get(key, nq) < t:
                        assert t == nq - 1 and all((tt, h) in seen for h in cur for tt in range(nq))
                        cur.clear()
                    cur.add(bh)
                assert last.get(key, nq) >= t or t == nq - 1
            else:
                assert last.get(key, nq) >= t  # longest first over the whole grid
            last[key] = t
    assert len(seen) == G
    if causal:
        t0, _ = ea.attn_fwd_workgroup_tile(B, H, S, D, causal, 0, 0)
        assert t0 == nq - 1
    with pytest.raises(_lib.AttnError):
        ea.attn_fwd_workgroup_tile(B, H, S, D, causal, 0, G)


def test_causal_map_chunks_heads_within_the_l2_budget():
    # B=16 H=32 S=1024 D=64: K and V of a head are 256 KiB, so a chunk holds
    # 16 heads (4 MiB); every XCD's first 16 * 8 workgroups cover 16 heads
    B, H, S, D = 16, 32, 1024, 64
    for x in range(8):
        first = {ea.attn_fwd_workgroup_tile(B, H, S, D, True, 0, wg)[1] for wg in range(x, 8 * 128, 8)}
        assert len(first) == 16 and all(h % 8 == x for h in first)


def test_causal_map_balances_each_xcd():
    # B=4 H=16 S=2048 D=128 causal: 64 x 8 tiles, tile t costs t + 1. Greedy
    # list scheduling of each XCD's workgroups, in id order, onto 32 CUs that
    # each hold one workgroup at a time gives every CU the same total (with
    # 1 MiB of K and V per head, a chunk is 4 of the XCD's 8 heads).
    B, H, S, D = 4, 16, 2048, 128
    p = ea.attn_fwd_plan(B, H, S, D, True, 1)
    G = p["num_workgroups"]
    for x in range(8):
        cus = [0] * 32
        for wg in range(x, G, 8):
            t, _ = ea.attn_fwd_workgroup_tile(B, H, S, D, True, 1, wg)
            i = min(range(32), key=lambda c: cus[c])
            cus[i] += t + 1
        assert max(cus) == min(cus)


def test_workgroup_map_keeps_heads_on_one_xcd():
    # 512 workgroups (16 tiles x 32 heads): XCD x = wg % 8 owns heads 4x..4x+3
    B, H, S, D = 2, 16, 4096, 128
    for wg in range(512):
        _, bh = ea.attn_fwd_workgroup_tile(B, H, S, D, False, 0, wg)
        assert bh // 4 == wg % 8


def plain_map(G, nq, causal, hchunk, g):
    """The documented workgroup order with plain integer division (the
    library divides by multiplying with reciprocals fixed on the host)."""
    X = 8
    xcd, slot = g % X, g // X
    if causal:
        heads = G // nq
        hc = heads if hchunk > heads else max(hchunk, 0)
        if heads % X or hc == 0:
            return nq - 1 - g // heads, g % heads
        hx = heads // X
        c = min(hc, hx)
        chunk = slot // (c * nq)
        r = slot - chunk * c * nq
        cw = min(hx - chunk * c, c)
        return nq - 1 - r // cw, (chunk * c + r % cw) * X + xcd
    base, rem = G // X, G % X
    logical = xcd * base + min(xcd, rem) + slot
    return logical % nq, logical // nq


# grids up to 2^30 workgroups (quotients of numerators near 2^31), tile
# counts and head counts that are and are not powers of two, short last
# chunks, heads not a multiple of 8
@pytest.mark.parametrize("B,H,S,D", [(1, 1 << 23, 16384, 64), (1, 8388613, 8192, 64), (7, 3 << 18, 4000, 128),
                                     (5, 77, 100000, 256), (2, 1 << 20, 2048, 128), (1, 1 << 22, 8191, 256),
                                     (3, 1000, 5000, 64), (1, 24, 300, 128)])
@pytest.mark.parametrize("causal", [False, True])
def test_workgroup_map_matches_plain_division(B, H, S, D, causal):
    import random
    p = ea.attn_fwd_plan(B, H, S, D, causal, 0)
    G, nq = p["num_workgroups"], p["num_q_tiles"]
    hchunk = max(1, (4 << 20) // (4 * S * D))
    rng = random.Random(G)
    ids = list(range(min(G, 300))) + list(range(max(0, G - 300), G)) + [rng.randrange(G) for _ in range(600)]
    for wg in ids:
        assert ea.attn_fwd_workgroup_tile(B, H, S, D, causal, 0, wg) == plain_map(G, nq, causal, hchunk, wg), wg


FAKE = 0x10000  # never dereferenced: every case below fails before any HIP call


def call(q=FAKE, k=FAKE + 0x100000, v=FAKE + 0x200000, o=FAKE + 0x300000, lse=FAKE + 0x400000,
         B=1, H=1, S=16, D=64, scale=0.125, causal=0, dtype=0):
    return _lib.attn_fwd(q, k, v, o, lse, B, H, S, D, scale, causal, dtype, 0)


@pytest.mark.parametrize("kwargs,status,word", [
    (dict(q=0), 1, "NULL"),
    (dict(lse=0), 1, "NULL"),
    (dict(B=-1), 2, "B, H and S"),
    (dict(S=-5), 2, "B, H and S"),
    (dict(S=1 << 30), 2, "too large"),
    (dict(S=(1 << 24) + 1, D=64), 2, "too large"),
    (dict(B=1 << 40, H=1 << 20), 2, "overflow"),
    (dict(D=96), 3, "head_dim"),
    (dict(dtype=2), 4, "dtype"),
    (dict(q=FAKE + 8), 5, "16-byte"),
    (dict(o=FAKE + 0x300002), 5, "16-byte"),
    (dict(lse=FAKE + 0x400002), 5, "4-byte"),
    (dict(scale=float("nan")), 6, "scale"),
    (dict(scale=float("inf")), 6, "scale"),
    (dict(scale=float("-inf")), 6, "scale"),
    (dict(o=FAKE), 7, "overlaps"),
    (dict(o=FAKE + 0x100000 + 16), 7, "overlaps"),
    (dict(lse=FAKE + 0x300000 + 64), 7, "overlaps"),
    (dict(lse=FAKE + 16), 7, "overlaps"),
])
def test_invalid_arguments_rejected_before_launch(kwargs, status, word):
    st = call(**kwargs)
    assert st == status, (st, _lib.last_error())
    assert word.lower() in _lib.last_error().lower()


def test_empty_inputs_are_a_noop():
    for kw in (dict(B=0), dict(H=0), dict(S=0)):
        assert call(q=0, k=0, v=0, o=0, lse=0, **kw) == 0
        assert _lib.last_error() == ""


def test_qkv_may_alias_each_other():
    # q == k == v is legal (read-only); validation passes and only the device
    # check (no GPU here) can fail
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("would launch on a real GPU with fake pointers")
    st = call(q=FAKE, k=FAKE, v=FAKE)
    assert st == 8, _lib.last_error()


def test_no_gpu_reports_unsupported_device():
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present")
    assert call() == 8
    assert "device" in _lib.last_error()


def test_any_finite_scale_passes_the_checks():
    # the page's sm_scale is a plain f32: zero and negative scales are valid
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("would launch on a real GPU with fake pointers")
    for sc in (-0.5, -0.0, 0.0, -1e30, 3.0e38):
        assert call(scale=sc) == 8, (sc, _lib.last_error())
        assert scall(scale=sc) == 8, (sc, _lib.last_error())


# --------------------------------------------------------------------------
# attn_fwd_strided: argument checks (all before any HIP call)
# --------------------------------------------------------------------------
def scall(q=FAKE, k=FAKE + 0x1000000, v=FAKE + 0x2000000, o=FAKE + 0x3000000, lse=FAKE + 0x4000000,
          B=1, H=2, Sq=16, Skv=24, D=64, qs=None, ks=None, vs=None, os_=None, scale=0.125, causal=0,
          dtype=0):
    return _lib.attn_fwd_strided(q, k, v, o, lse, B, H, Sq, Skv, D, qs, ks, vs, os_, scale, causal,
                                 dtype, 0)


@pytest.mark.parametrize("kwargs,status,word", [
    (dict(Sq=-1), 2, "Sq and Skv"),
    (dict(Skv=-3), 2, "Sq and Skv"),
    (dict(Skv=1 << 30), 2, "too large"),
    (dict(D=96), 3, "head_dim"),
    (dict(dtype=7), 4, "dtype"),
    (dict(k=0), 1, "NULL"),
    (dict(qs=(2048, 1024, 56)), 10, "shorter than a row"),
    (dict(vs=(3072, -1536, 64)), 10, ">= 0"),
    (dict(ks=(3072, 1536, 68)), 5, "multiples of 8"),
    (dict(os_=(2048, 1028, 64)), 5, "multiples of 8"),
    (dict(qs=(0, 0, 1 << 31)), 2, "2 gib"),
    (dict(os_=(2048, 512, 64)), 7, "o strides"),        # head 1 starts inside head 0's 16 rows
    (dict(os_=(2048, 32, 128)), 7, "o strides"),        # head 1 starts in the middle of a row of head 0
    (dict(o=FAKE + 64), 7, "overlaps"),
    (dict(lse=FAKE + 0x2000000 + 64), 7, "overlaps"),
    (dict(scale=float("nan")), 6, "scale"),
])
def test_strided_invalid_arguments_rejected_before_launch(kwargs, status, word):
    st = scall(**kwargs)
    assert st == status, (st, _lib.last_error())
    assert word.lower() in _lib.last_error().lower()


def test_strided_empty_query_is_a_noop():
    assert scall(q=0, k=0, v=0, o=0, lse=0, Sq=0) == 0
    assert scall(q=0, k=0, v=0, o=0, lse=0, B=0) == 0


def test_strided_valid_layouts_reach_the_device_check():
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("would launch on a real GPU with fake pointers")
    # [B,S,H,D] views (row stride H*D), padded rows, a size-1 batch whose
    # (unaligned) batch stride never addresses anything, and Skv = 0
    B, H, Sq, Skv, D = 2, 4, 16, 24, 64
    for kw in (dict(qs=(Sq * H * D, D, H * D), ks=(Skv * H * D, D, H * D), vs=(Skv * H * D, D, H * D),
                    os_=(Sq * H * D, D, H * D)),
               dict(qs=(H * Sq * 72, Sq * 72, 72), os_=(H * Sq * 72, Sq * 72, 72)),
               dict(B=1, qs=(3, Sq * D, D)),
               dict(Skv=0)):
        args = dict(B=B, H=H, Sq=Sq, Skv=Skv, D=D)
        args.update(kw)
        assert scall(**args) == 8, _lib.last_error()


# --------------------------------------------------------------------------
# attn_bwd: argument checks (all before any HIP call)
# --------------------------------------------------------------------------
MB_ = 0x1000000


def bcall(q=FAKE, k=FAKE + MB_, v=FAKE + 2 * MB_, o=FAKE + 3 * MB_, lse=FAKE + 4 * MB_, do=FAKE + 5 * MB_,
          dq=FAKE + 6 * MB_, dk=FAKE + 7 * MB_, dv=FAKE + 8 * MB_, delta=FAKE + 9 * MB_, B=1, H=2, Sq=16,
          Skv=24, D=64, scale=0.125, causal=0, dtype=0):
    return _lib.attn_bwd(q, k, v, o, lse, do, dq, dk, dv, delta, B, H, Sq, Skv, D, scale, causal, dtype, 0)


@pytest.mark.parametrize("kwargs,status,word", [
    (dict(Sq=-1), 2, ">= 0"),
    (dict(Skv=1 << 30), 2, "too large"),
    (dict(D=80), 3, "head_dim"),
    (dict(dtype=2), 4, "dtype"),
    (dict(scale=float("nan")), 6, "scale"),
    (dict(do=0), 1, "NULL"),
    (dict(delta=0), 1, "NULL"),
    (dict(dk=0), 1, "NULL"),
    (dict(dq=FAKE + 6 * MB_ + 8), 5, "16-byte"),
    (dict(lse=FAKE + 4 * MB_ + 2), 5, "4-byte"),
    (dict(dk=FAKE + 6 * MB_ + 64), 7, "each other"),           # dk inside dq
    (dict(delta=FAKE + 8 * MB_), 7, "each other"),             # delta on dv
    (dict(dv=FAKE + 5 * MB_ + 16), 7, "must not overlap q"),   # dv inside dO
    (dict(dq=FAKE + 4 * MB_), 7, "must not overlap q"),        # dq on lse
])
def test_bwd_invalid_arguments_rejected_before_launch(kwargs, status, word):
    st = bcall(**kwargs)
    assert st == status, (st, _lib.last_error())
    assert word.lower() in _lib.last_error().lower()


def test_bwd_empty_calls():
    assert bcall(B=0) == 0
    assert bcall(Sq=0, Skv=0, q=0, k=0, v=0, o=0, lse=0, do=0, dq=0, dk=0, dv=0, delta=0) == 0


def test_bwd_null_tensors_without_elements_reach_the_device_check():
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("would launch on a real GPU with fake pointers")
    # no queries: q, o, dO, lse, dq, delta are never touched; no keys: k, v, dk, dv
    assert bcall(Sq=0, q=0, o=0, lse=0, do=0, dq=0, delta=0) == 8, _lib.last_error()
    assert bcall(Skv=0, k=0, v=0, dk=0, dv=0) == 8, _lib.last_error()
    assert bcall(k=FAKE, v=FAKE, q=FAKE, o=FAKE, do=FAKE) == 8, _lib.last_error()  # inputs may alias


# --------------------------------------------------------------------------
# attn_fwd_unfused (the comparator): workspace size and argument checks
# --------------------------------------------------------------------------
def test_unfused_workspace_bytes():
    # per head S rows of fp32 padded to 4 elements, then (256-byte aligned)
    # S rows of 16-bit padded to 8, then (aligned) the fp32 O and one fp32 per row
    p_end = 512 + 2 * 5 * 8 * 2
    o_off = (p_end + 255) // 256 * 256
    assert _lib.attn_fwd_unfused_workspace_bytes(1, 2, 5, 64) == o_off + 2 * 5 * 64 * 4 + 2 * 5 * 4
    n = 2 * 16 * 4096
    assert _lib.attn_fwd_unfused_workspace_bytes(2, 16, 4096, 128) == n * 4096 * 6 + n * 128 * 4 + n * 4
    assert _lib.attn_fwd_unfused_workspace_bytes(0, 2, 5, 64) == 0
    assert _lib.attn_fwd_unfused_workspace_bytes(-1, 2, 5, 64) == -1
    assert _lib.attn_fwd_unfused_workspace_bytes(1, 2, 5, 96) == -1
    assert _lib.attn_fwd_unfused_workspace_bytes(1 << 40, 1 << 10, 1 << 20, 64) == -1


def ucall(q=FAKE, k=FAKE + MB_, v=FAKE + 2 * MB_, o=FAKE + 3 * MB_, lse=FAKE + 4 * MB_, ws=FAKE + 16 * MB_,
          wsb=1 << 20, B=1, H=2, S=16, D=64, scale=0.125, causal=0, dtype=0):
    return _lib.attn_fwd_unfused(q, k, v, o, lse, ws, wsb, B, H, S, D, scale, causal, dtype, 0)


@pytest.mark.parametrize("kwargs,status,word", [
    (dict(S=-2), 2, ">= 0"),
    (dict(D=48), 3, "head_dim"),
    (dict(ws=0), 1, "NULL"),
    (dict(ws=FAKE + 16 * MB_ + 8), 5, "16-byte"),
    (dict(wsb=100), 10, "needed"),
    (dict(ws=FAKE + 3 * MB_), 7, "workspace overlaps"),
    (dict(o=FAKE + 64), 7, "o overlaps"),
])
def test_unfused_invalid_arguments_rejected_before_launch(kwargs, status, word):
    st = ucall(**kwargs)
    assert st == status, (st, _lib.unfused_last_error())
    assert word.lower() in _lib.unfused_last_error().lower()


def test_unfused_valid_call_reaches_the_device_check():
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("would launch on a real GPU with fake pointers")
    assert ucall() == 8, _lib.unfused_last_error()
    assert ucall(B=0, q=0, k=0, v=0, o=0, lse=0, ws=0, wsb=0) == 0
    assert ucall(scale=-0.25) == 8, _lib.unfused_last_error()


# --------------------------------------------------------------------------
# attn_fwd_variant: the A/B schedules
# --------------------------------------------------------------------------
def vcall(variant, D=64, B=1, H=2, S=16, q=FAKE, o=FAKE + 3 * MB_, lse=FAKE + 4 * MB_):
    return _lib.attn_fwd_variant(q, q, q, o, lse, B, H, S, D, 0.125, 0, 0, variant, 0)


@pytest.mark.parametrize("variant,D", [(-1, 64), (7, 64), (7, 256), (1, 256), (4, 256)])
def test_variant_out_of_range(variant, D):
    assert vcall(variant, D) == 10
    assert "variant" in _lib.last_error()


def test_variants_reach_the_device_check():
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("would launch on a real GPU with fake pointers")
    for v in range(7):
        for D in (64, 128):
            assert vcall(v, D) == 8, _lib.last_error()
    for v in (0, 5, 6):
        assert vcall(v, 256) == 8, _lib.last_error()
    assert vcall(3, 64, B=0) == 0  # empty


def bscall(strides, **kw):
    args = dict(q=FAKE, k=FAKE + MB_, v=FAKE + 2 * MB_, o=FAKE + 3 * MB_, lse=FAKE + 4 * MB_, do=FAKE + 5 * MB_,
                dq=FAKE + 6 * MB_, dk=FAKE + 7 * MB_, dv=FAKE + 8 * MB_, delta=FAKE + 9 * MB_, B=1, H=2, Sq=16,
                Skv=24, D=64)
    args.update(kw)
    st = [strides.get(n) for n in ("q", "k", "v", "o", "do", "dq", "dk", "dv")]
    return _lib.attn_bwd_strided(args["q"], args["k"], args["v"], args["o"], args["lse"], args["do"], args["dq"],
                                 args["dk"], args["dv"], args["delta"], args["B"], args["H"], args["Sq"],
                                 args["Skv"], args["D"], st, 0.125, 0, 0, 0)


@pytest.mark.parametrize("strides,status,word", [
    ({"k": (3072, -1536, 64)}, 10, ">= 0"),
    ({"do": (2048, 1024, 60)}, 10, "shorter than a row"),
    ({"dv": (3072, 1536, 68)}, 5, "multiples of 8"),
    ({"dq": (2048, 512, 64)}, 7, "dq strides"),        # head 1 inside head 0's 16 rows
    ({"dk": (3072, 32, 128)}, 7, "dk strides"),
])
def test_bwd_strided_invalid_arguments(strides, status, word):
    st = bscall(strides)
    assert st == status, (st, _lib.last_error())
    assert word.lower() in _lib.last_error().lower()


def test_bwd_strided_extent_aliasing():
    # dq starts past lse, but its second head (16 MiB on) lies inside dO's region
    st = bscall({"dq": (1 << 24, 1 << 23, 64)}, dq=FAKE + 4 * MB_ + 4096)
    assert st == 7 and "overlap" in _lib.last_error()


def test_bwd_strided_valid_layouts_reach_the_device_check():
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("would launch on a real GPU with fake pointers")
    H, Sq, Skv, D = 2, 16, 24, 64
    bshd_q = (Sq * H * D, D, H * D)
    bshd_k = (Skv * H * D, D, H * D)
    layouts = {"q": bshd_q, "o": bshd_q, "do": bshd_q, "dq": bshd_q, "k": bshd_k, "v": bshd_k, "dk": bshd_k,
               "dv": bshd_k}
    assert bscall(layouts) == 8, _lib.last_error()
    assert bscall({}) == 8, _lib.last_error()


# --------------------------------------------------------------------------
# attn_bwd_noalloc: the scratch bound is checked before any HIP call
# --------------------------------------------------------------------------
def nacall(B=1, H=2, Sq=16, Skv=24, D=64, gap=MB_):
    p = [FAKE + i * gap for i in range(9)]
    return _lib.attn_bwd_noalloc(*p, B, H, Sq, Skv, D, 0.125, 0, 0, 0)


def test_noalloc_rejects_more_rows_than_the_scratch_holds():
    assert nacall(B=1, H=1, Sq=(1 << 22) + 1, Skv=8) == 10
    assert "scratch" in _lib.last_error()
    assert nacall(B=4, H=1 << 10, Sq=1 << 10 | 1, Skv=8) == 10
    assert nacall(D=96) == 3  # the ordinary checks still apply


def test_noalloc_valid_call_reaches_the_device_check():
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("would launch on a real GPU with fake pointers")
    assert nacall() == 8, _lib.last_error()
    assert nacall(B=1, H=1, Sq=1 << 22, Skv=8, gap=1 << 30) == 8, _lib.last_error()
    assert nacall(B=0) == 0
