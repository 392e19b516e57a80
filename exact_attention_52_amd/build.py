"""Build libattn.so (the C-ABI library with the gfx950 kernels) and
libattn_unfused.so (the unfused comparator) in-tree."""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libattn.so")
UNFUSED_LIB = os.path.join(PKG, "libattn_unfused.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _c(name):
    return os.path.join(CSRC, name)


# libattn.so: the fused forward, its schedule variants and the backward.
SOURCES = [_c("attn_api.hip"), _c("attn_bwd.hip"), _c("attn_variants.hip")]
HEADERS = [_c("attn_fwd_kernel.hpp"), _c("attn_bwd_kernel.hpp"), _c("attn_bwd.hpp"), _c("attn_variants.hpp"),
           _c("attn_grid.hpp"), _c("attn_common.hpp"), os.path.join(INCLUDE, "attn.h")]
# libattn_unfused.so: the unfused comparator, the only code that uses the
# vendor BLAS, in a library of its own.
UNFUSED_SOURCES = [_c("attn_unfused.hip")]
UNFUSED_HEADERS = [_c("attn_unfused.hpp"), _c("attn_common.hpp"), os.path.join(INCLUDE, "attn.h"),
                   os.path.join(INCLUDE, "attn_unfused.h")]

FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC",
    "-Wall", "-Werror", "-Wno-unused-command-line-argument",
    # keep the compiler from emitting packed-fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# Per-source flags.  MFMA accumulators in VGPRs: left to its heuristics the
# compiler parks accumulators in AGPRs and copies them to VGPRs and back
# around loop boundaries (the forward's D=256 output accumulator on every key
# tile: the rescale multiplies it on the VALU, which cannot address AGPRs; the
# backward's dK/dV accumulators at every loop header); in VGPR form the forward
# D=256 kernel fits in 249 VGPRs with no copies and the D=64/128 dK/dV kernels
# fit two waves per SIMD.
SOURCE_FLAGS = {
    "attn_api.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form=1"],
    "attn_bwd.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form=1"],
    "attn_unfused.hip": [],
    "attn_variants.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form=1"],
}
# the unfused comparator's GEMMs are the vendor library's
UNFUSED_LINK_LIBS = ["-L/opt/rocm/lib", "-lrocblas"]


def _run(cmd, name):
    proc = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (proc.stdout + proc.stderr).splitlines()
            if "packed-fp32-ops' is not a recognized feature" not in ln]
    if proc.returncode != 0:
        sys.stderr.write("\n".join(msgs) + "\n")
        raise RuntimeError(f"hipcc failed building {name}")
    if msgs:
        sys.stderr.write("\n".join(msgs) + "\n")


def _link(sources, out, link_libs, extra_flags, name):
    """Compile each source to an object (with its own flags) and link them."""
    tmp = out + ".tmp"
    with tempfile.TemporaryDirectory() as d:
        objs = []
        for src in sources:
            obj = os.path.join(d, os.path.basename(src) + ".o")
            _run([HIPCC, *FLAGS, *SOURCE_FLAGS[os.path.basename(src)], *extra_flags,
                  "-I" + INCLUDE, "-I" + CSRC, "-c", "-o", obj, src], name)
            objs.append(obj)
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs, *link_libs], name)
    os.replace(tmp, out)
    return out


def build(out: str = LIB, extra_flags=(), unfused_out: str = UNFUSED_LIB) -> str:
    """Build libattn.so and libattn_unfused.so; returns the path of the first."""
    _link(SOURCES, out, [], extra_flags, "libattn.so")
    if unfused_out:
        _link(UNFUSED_SOURCES, unfused_out, UNFUSED_LINK_LIBS, extra_flags, "libattn_unfused.so")
    return out


def is_stale() -> bool:
    """Whether either library is missing or older than one of its sources."""
    for out, deps in ((LIB, SOURCES + HEADERS), (UNFUSED_LIB, UNFUSED_SOURCES + UNFUSED_HEADERS)):
        if not os.path.exists(out):
            return True
        t = os.path.getmtime(out)
        if any(os.path.getmtime(p) > t for p in deps):
            return True
    return False


if __name__ == "__main__":
    print(build())
