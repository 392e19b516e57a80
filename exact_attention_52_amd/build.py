"""Build libattn.so (the C-ABI library with the gfx950 kernels) in-tree."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libattn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = [os.path.join(CSRC, "attn_api.hip")]
HEADERS = [os.path.join(CSRC, "attn_fwd_kernel.hpp"), os.path.join(INCLUDE, "attn.h")]

FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-command-line-argument",
    # keep the compiler from emitting packed-fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: left to its heuristics the compiler parks the
    # D=256 output accumulator in AGPRs and copies all of it to VGPRs and back
    # on every key tile (the rescale multiplies it on the VALU, which cannot
    # address AGPRs); in VGPR form the kernel fits in 249 VGPRs with no copies
    "-mllvm", "--amdgpu-mfma-vgpr-form=1",
]


def build(out: str = LIB, extra_flags=()) -> str:
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *extra_flags, "-I" + INCLUDE, "-I" + CSRC, "-o", tmp, *SOURCES]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (proc.stdout + proc.stderr).splitlines()
            if "packed-fp32-ops' is not a recognized feature" not in ln]
    if proc.returncode != 0:
        sys.stderr.write("\n".join(msgs) + "\n")
        raise RuntimeError("hipcc failed building libattn.so")
    if msgs:
        sys.stderr.write("\n".join(msgs) + "\n")
    os.replace(tmp, out)
    return out


def is_stale(out: str = LIB) -> bool:
    if not os.path.exists(out):
        return True
    t = os.path.getmtime(out)
    return any(os.path.getmtime(p) > t for p in SOURCES + HEADERS)


if __name__ == "__main__":
    print(build())
