"""Compile the HIP library (gfx950) into all_reduce_residual_amd/libar_fused.so.

The kernels are instantiated per element type in separate translation units (csrc/inst_*.hip);
they compile in parallel and link with the host side (csrc/ar_fused.hip) into one shared
library.
"""
from __future__ import annotations

import os
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SOURCES = ["ar_fused.hip", "inst_bf16.hip", "inst_f16.hip", "inst_f32.hip"]
LIB = os.path.join(PKG, "libar_fused.so")
# The benchmark's streaming-bandwidth calibration (include/ar_probe.h), a library of its own.
PROBE_SOURCES = ["stream_probe.hip"]
PROBE_LIB = os.path.join(PKG, "libar_probe.so")
ARCH = "gfx950"

# -packed-fp32-ops (device code only): keep the compiler from fusing binary32 adds/multiplies
# into packed two-lane instructions; every add of the rank chain is a plain v_add_f32.  Each
# source is compiled in two passes -- the gfx950 code with that feature into a code-object
# bundle, then the host code with the bundle embedded -- so the host compiler never sees the
# target feature (it is not one of the host target's).
COMMON_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
                "-Wno-unused-command-line-argument"]
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# The device pass's flags in one list (the assembly checks compile device code with them).
HIPCC_FLAGS = COMMON_FLAGS + DEVICE_FLAGS


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def build(extra_flags=(), out: str = LIB, jobs: int = 0, probe: bool = True) -> str:
    """Build the library (and, with `probe`, the calibration probe library) and return the
    library's path (always recompiles)."""
    inc = "-I" + os.path.join(ROOT, "include")
    sources = SOURCES + (PROBE_SOURCES if probe else [])
    jobs = jobs or min(len(sources), os.cpu_count() or 1)
    with tempfile.TemporaryDirectory(prefix="ar_build_") as tmpdir:
        def compile_one(src):
            stem = os.path.join(tmpdir, os.path.splitext(src)[0])
            path = os.path.join(CSRC, src)
            subprocess.run([hipcc()] + COMMON_FLAGS + DEVICE_FLAGS + list(extra_flags) +
                           [inc, "--cuda-device-only", "-c", "-o", stem + ".hipfb", path],
                           check=True)
            subprocess.run([hipcc()] + COMMON_FLAGS + list(extra_flags) +
                           [inc, "--cuda-host-only", "-Xclang", "-fcuda-include-gpubinary",
                            "-Xclang", stem + ".hipfb", "-c", "-o", stem + ".o", path],
                           check=True)
            return stem + ".o"

        def link(objs, target):
            tmp = target + ".tmp%d" % os.getpid()
            subprocess.run([hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] +
                           objs, check=True)
            os.replace(tmp, target)

        with ThreadPoolExecutor(max_workers=jobs) as pool:
            objs = list(pool.map(compile_one, sources))
        link(objs[:len(SOURCES)], out)
        if probe:
            link(objs[len(SOURCES):], PROBE_LIB)
    return out


if __name__ == "__main__":
    print(build())
