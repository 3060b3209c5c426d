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
# The benchmark's probes (bench_probes/ar_probe.h: the streaming-bandwidth calibration and the
# phase timing), a library of their own that the all-reduce library does not contain.
PROBES = os.path.join(PKG, "bench_probes")
PROBE_SOURCES = ["stream_probe.hip", "phase_probe.hip"]
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
    """Build the library (and, with `probe`, the benchmark's probe library) and return the
    library's path (always recompiles)."""
    inc = "-I" + os.path.join(ROOT, "include")
    sources = [os.path.join(CSRC, x) for x in SOURCES]
    if probe:
        sources += [os.path.join(PROBES, x) for x in PROBE_SOURCES]
    jobs = jobs or min(len(sources), os.cpu_count() or 1)
    with tempfile.TemporaryDirectory(prefix="ar_build_") as tmpdir:
        def compile_one(path):
            stem = os.path.join(tmpdir, os.path.splitext(os.path.basename(path))[0])
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
