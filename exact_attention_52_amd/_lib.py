"""ctypes binding of libattn.so (the C ABI of include/attn.h) and of
libattn_unfused.so (include/attn_unfused.h), one Python name per exported
symbol.  Argument marshalling only; every step of the attention
runs in the library's gfx950 kernels."""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn.so")
ABI_VERSION = 6

ATTN_F16, ATTN_BF16 = 0, 1
STATUS = {
    0: "ATTN_OK", 1: "ATTN_ERR_NULL_PTR", 2: "ATTN_ERR_BAD_SHAPE",
    3: "ATTN_ERR_UNSUPPORTED_HEAD_DIM", 4: "ATTN_ERR_UNSUPPORTED_DTYPE",
    5: "ATTN_ERR_MISALIGNED", 6: "ATTN_ERR_BAD_SCALE", 7: "ATTN_ERR_ALIASING",
    8: "ATTN_ERR_UNSUPPORTED_DEVICE", 9: "ATTN_ERR_LAUNCH", 10: "ATTN_ERR_BAD_ARGUMENT",
}
UNFUSED_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn_unfused.so")
EXPORTS = ("attn_fwd", "attn_fwd_strided", "attn_fwd_variant", "attn_bwd", "attn_bwd_strided", "attn_bwd_noalloc",
           "attn_fwd_plan", "attn_fwd_workgroup_tile", "attn_status_string", "attn_last_error", "attn_abi_version")
UNFUSED_EXPORTS = ("attn_fwd_unfused", "attn_fwd_unfused_workspace_bytes", "attn_unfused_last_error")


class AttnError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status
        self.detail = detail


class Plan(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "block_m", "block_n", "kv_stages", "waves_q", "waves_k",
        "threads_per_workgroup", "lds_bytes", "num_q_tiles", "num_workgroups")]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


_lib = None


def load():
    """Load libattn.so; raise loudly if it is missing (no fallback exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m exact_attention_52_amd.build` "
            "(or __graft_entry__.build()); there is no CPU or fallback path")
    lib = ctypes.CDLL(LIB_PATH)
    i64, vp, ci, cf = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, cf, ci, ci, vp]
    lib.attn_fwd.restype = ci
    p64 = ctypes.POINTER(i64)
    lib.attn_fwd_strided.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, p64, p64, p64, p64,
                                     cf, ci, ci, vp]
    lib.attn_fwd_strided.restype = ci
    lib.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, cf, ci, ci, vp]
    lib.attn_bwd.restype = ci
    lib.attn_bwd_strided.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                     p64, p64, p64, p64, p64, p64, p64, p64, cf, ci, ci, vp]
    lib.attn_bwd_strided.restype = ci
    lib.attn_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, cf, ci, ci, vp]
    lib.attn_bwd_noalloc.restype = ci
    lib.attn_fwd_variant.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, cf, ci, ci, ci, vp]
    lib.attn_fwd_variant.restype = ci
    lib.attn_fwd_plan.argtypes = [i64, i64, i64, i64, ci, ci, ctypes.POINTER(Plan)]
    lib.attn_fwd_plan.restype = ci
    lib.attn_fwd_workgroup_tile.argtypes = [i64, i64, i64, i64, ci, ci, i64,
                                            ctypes.POINTER(i64), ctypes.POINTER(i64)]
    lib.attn_fwd_workgroup_tile.restype = ci
    lib.attn_status_string.argtypes = [ci]
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_last_error.argtypes = []
    lib.attn_last_error.restype = ctypes.c_char_p
    lib.attn_abi_version.argtypes = []
    lib.attn_abi_version.restype = ci
    if lib.attn_abi_version() != ABI_VERSION:
        raise ImportError(f"libattn.so ABI {lib.attn_abi_version()} != expected {ABI_VERSION}")
    _lib = lib
    return lib


_unfused = None


def load_unfused():
    """Load libattn_unfused.so, the unfused comparator (its own library: the
    fused libattn.so links no vendor BLAS); raise loudly if it is missing."""
    global _unfused
    if _unfused is not None:
        return _unfused
    load()  # the comparator shares libattn.so's status codes; both are built together
    if not os.path.exists(UNFUSED_LIB_PATH):
        raise ImportError(
            f"{UNFUSED_LIB_PATH} is missing: build it with `python -m exact_attention_52_amd.build` "
            "(or __graft_entry__.build()); there is no CPU or fallback path")
    lib = ctypes.CDLL(UNFUSED_LIB_PATH)
    i64, vp, ci, cf = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.attn_fwd_unfused.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, cf, ci, ci, vp]
    lib.attn_fwd_unfused.restype = ci
    lib.attn_fwd_unfused_workspace_bytes.argtypes = [i64, i64, i64, i64]
    lib.attn_fwd_unfused_workspace_bytes.restype = i64
    lib.attn_unfused_last_error.argtypes = []
    lib.attn_unfused_last_error.restype = ctypes.c_char_p
    _unfused = lib
    return lib


def unfused_last_error() -> str:
    return load_unfused().attn_unfused_last_error().decode()


def check_unfused(status: int) -> None:
    if status != 0:
        raise AttnError(status, unfused_last_error())


def last_error() -> str:
    return load().attn_last_error().decode()


def status_string(status: int) -> str:
    return load().attn_status_string(int(status)).decode()


def check(status: int) -> None:
    if status != 0:
        raise AttnError(status, last_error())


def attn_fwd(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, S: int, D: int,
             scale: float, causal: bool, dtype: int, stream: int) -> int:
    """Raw call: device pointers as ints; returns the status code."""
    return load().attn_fwd(q, k, v, o, lse, B, H, S, D, float(scale), int(bool(causal)),
                           int(dtype), stream)


def _strides(st):
    if st is None:
        return None
    st = tuple(int(x) for x in st)
    if len(st) != 3:
        raise ValueError("strides are (batch, head, row) in elements")
    return (ctypes.c_int64 * 3)(*st)


def attn_fwd_strided(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, Sq: int, Skv: int,
                     D: int, q_strides, k_strides, v_strides, o_strides, scale: float, causal: bool,
                     dtype: int, stream: int) -> int:
    """Raw call: device pointers as ints, strides as (batch, head, row) element
    triples or None (contiguous); returns the status code."""
    return load().attn_fwd_strided(q, k, v, o, lse, B, H, Sq, Skv, D, _strides(q_strides),
                                   _strides(k_strides), _strides(v_strides), _strides(o_strides),
                                   float(scale), int(bool(causal)), int(dtype), stream)


def attn_bwd(q: int, k: int, v: int, o: int, lse: int, do: int, dq: int, dk: int, dv: int, delta: int,
             B: int, H: int, Sq: int, Skv: int, D: int, scale: float, causal: bool, dtype: int,
             stream: int) -> int:
    """Raw call: device pointers as ints; returns the status code."""
    return load().attn_bwd(q, k, v, o, lse, do, dq, dk, dv, delta, B, H, Sq, Skv, D, float(scale),
                           int(bool(causal)), int(dtype), stream)


def attn_bwd_noalloc(q: int, k: int, v: int, o: int, lse: int, do: int, dq: int, dk: int, dv: int,
                     B: int, H: int, Sq: int, Skv: int, D: int, scale: float, causal: bool, dtype: int,
                     stream: int) -> int:
    """Raw call: attn_bwd with D_i in the library's own device scratch (no
    allocation, no delta argument); device pointers as ints; returns the
    status code."""
    return load().attn_bwd_noalloc(q, k, v, o, lse, do, dq, dk, dv, B, H, Sq, Skv, D, float(scale),
                                   int(bool(causal)), int(dtype), stream)


def attn_bwd_strided(q: int, k: int, v: int, o: int, lse: int, do: int, dq: int, dk: int, dv: int, delta: int,
                     B: int, H: int, Sq: int, Skv: int, D: int, strides, scale: float, causal: bool,
                     dtype: int, stream: int) -> int:
    """Raw call: device pointers as ints; strides: 8 (batch, head, row) triples
    or None for (q, k, v, o, do, dq, dk, dv); returns the status code."""
    st = [_strides(x) for x in strides]
    if len(st) != 8:
        raise ValueError("8 stride triples: q, k, v, o, do, dq, dk, dv")
    return load().attn_bwd_strided(q, k, v, o, lse, do, dq, dk, dv, delta, B, H, Sq, Skv, D, *st,
                                   float(scale), int(bool(causal)), int(dtype), stream)


def attn_fwd_variant(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, S: int, D: int,
                     scale: float, causal: bool, dtype: int, variant: int, stream: int) -> int:
    """Raw call: attn_fwd with copy schedule `variant` (0..6); returns the status code."""
    return load().attn_fwd_variant(q, k, v, o, lse, B, H, S, D, float(scale), int(bool(causal)), int(dtype),
                                   int(variant), stream)


def attn_fwd_unfused(q: int, k: int, v: int, o: int, lse: int, workspace: int, workspace_bytes: int, B: int,
                     H: int, S: int, D: int, scale: float, causal: bool, dtype: int, stream: int) -> int:
    """Raw call: device pointers as ints; returns the status code."""
    return load_unfused().attn_fwd_unfused(q, k, v, o, lse, workspace, workspace_bytes, B, H, S, D, float(scale),
                                           int(bool(causal)), int(dtype), stream)


def attn_fwd_unfused_workspace_bytes(B: int, H: int, S: int, D: int) -> int:
    return int(load_unfused().attn_fwd_unfused_workspace_bytes(B, H, S, D))


def attn_fwd_plan(B: int, H: int, S: int, D: int, causal: bool, dtype: int) -> dict:
    p = Plan()
    check(load().attn_fwd_plan(B, H, S, D, int(bool(causal)), dtype, ctypes.byref(p)))
    return p.as_dict()


def attn_fwd_workgroup_tile(B: int, H: int, S: int, D: int, causal: bool, dtype: int, wg: int):
    t, bh = ctypes.c_int64(), ctypes.c_int64()
    check(load().attn_fwd_workgroup_tile(B, H, S, D, int(bool(causal)), dtype, wg,
                                         ctypes.byref(t), ctypes.byref(bh)))
    return t.value, bh.value
