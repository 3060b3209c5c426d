"""Compile the HIP library (gfx950) into all_reduce_residual_amd/libar_fused.so."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "ar_fused.hip")
LIB = os.path.join(PKG, "libar_fused.so")
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from fusing binary32 adds/multiplies into packed
# two-lane instructions; every add of the rank chain is a plain v_add_f32.
HIPCC_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def build(extra_flags=(), out: str = LIB) -> str:
    """Build the library and return its path (always recompiles)."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc()] + HIPCC_FLAGS + list(extra_flags) + [
        "-I" + os.path.join(ROOT, "include"), "-o", tmp, SRC]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
