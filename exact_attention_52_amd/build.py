"""Build libattn.so (the C-ABI library with the gfx950 kernels) in-tree."""
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
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = [os.path.join(CSRC, "attn_api.hip"), os.path.join(CSRC, "attn_bwd.hip"),
           os.path.join(CSRC, "attn_unfused.hip"), os.path.join(CSRC, "attn_variants.hip")]
HEADERS = [os.path.join(CSRC, "attn_fwd_kernel.hpp"), os.path.join(CSRC, "attn_bwd_kernel.hpp"),
           os.path.join(CSRC, "attn_bwd.hpp"), os.path.join(CSRC, "attn_unfused.hpp"),
           os.path.join(CSRC, "attn_variants.hpp"),
           os.path.join(INCLUDE, "attn.h")]

FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC",
    "-Wall", "-Wno-unused-command-line-argument",
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
LINK_LIBS = ["-L/opt/rocm/lib", "-lrocblas"]


def _run(cmd):
    proc = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (proc.stdout + proc.stderr).splitlines()
            if "packed-fp32-ops' is not a recognized feature" not in ln]
    if proc.returncode != 0:
        sys.stderr.write("\n".join(msgs) + "\n")
        raise RuntimeError("hipcc failed building libattn.so")
    if msgs:
        sys.stderr.write("\n".join(msgs) + "\n")


def build(out: str = LIB, extra_flags=()) -> str:
    """Compile each source to an object (with its own flags) and link them."""
    tmp = out + ".tmp"
    with tempfile.TemporaryDirectory() as d:
        objs = []
        for src in SOURCES:
            obj = os.path.join(d, os.path.basename(src) + ".o")
            _run([HIPCC, *FLAGS, *SOURCE_FLAGS[os.path.basename(src)], *extra_flags,
                  "-I" + INCLUDE, "-I" + CSRC, "-c", "-o", obj, src])
            objs.append(obj)
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs, *LINK_LIBS])
    os.replace(tmp, out)
    return out


def is_stale(out: str = LIB) -> bool:
    if not os.path.exists(out):
        return True
    t = os.path.getmtime(out)
    return any(os.path.getmtime(p) > t for p in SOURCES + HEADERS)


if __name__ == "__main__":
    print(build())
