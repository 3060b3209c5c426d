"""Code-generation check of the fused kernel's streaming loads (CPU only: hipcc cross-compiles the
gfx950 code to assembly, nothing runs).

The fused kernel is bandwidth-bound only if each thread has all loads of a rank batch in flight
together. The compiler's scheduler has twice turned an intended batch into one load per DRAM round
trip (`load, s_waitcnt vmcnt(0), load, ...`), correct but up to 2x slower, and tests that
compare results cannot see that. This test compiles the norm-kernel shapes the launch planner
picks for rows of whole vectors up to H = 8192 (one or two 16-byte vectors per thread with one
chain per batch: W <= 8, and W = 16 with one vector) for the three element types, and asserts
that no full wait (`s_waitcnt vmcnt(0)`) falls between two of a kernel's streaming loads.
"""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from all_reduce_residual_amd import _build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SHAPES = [(w, v) for w in (1, 2, 4, 8) for v in (1, 2)] + [(16, 1)]
TYPES = ("Bf16", "F16", "F32")


def _source() -> str:
    refs = []
    for t in TYPES:
        for w, v in SHAPES:
            refs.append("reinterpret_cast<const void*>(&arf::ar_norm_kernel<arf::%s, %d, %d, true>)"
                        % (t, w, v))
    return ('#include "ar_kernels.hpp"\n'
            "const void* const kNormKernels[] = {\n  " + ",\n  ".join(refs) + "};\n")


def _waits_between_streaming_loads(asm: str) -> dict:
    """Per kernel symbol: the number of s_waitcnt vmcnt(0) that lie between two streaming
    (non-temporal) global loads of its body."""
    out, name, nt, pending = {}, None, 0, False
    for line in asm.splitlines():
        m = re.match(r"^(_Z\S*ar_norm_kernel\S*):", line)
        if m:
            name, nt, pending = m.group(1), 0, False
            out[name] = 0
            continue
        if name is None:
            continue
        if "global_load" in line and " nt" in line:
            if pending:
                out[name] += 1
                pending = False
            nt += 1
        elif "s_waitcnt" in line and "vmcnt(0)" in line and nt > 0:
            pending = True
        elif "s_endpgm" in line:
            name = None
    return out


@pytest.fixture(scope="module")
def norm_asm():
    hipcc = _build.hipcc()
    if not (os.path.exists(hipcc) or shutil.which(hipcc)):
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory(prefix="ar_isa_") as d:
        src = os.path.join(d, "norm_shapes.hip")
        with open(src, "w") as f:
            f.write(_source())
        asm = os.path.join(d, "norm_shapes.s")
        flags = [x for x in _build.HIPCC_FLAGS if x != "-fPIC"]
        subprocess.run([hipcc] + flags + ["-I" + os.path.join(ROOT, "include"),
                                          "-I" + _build.CSRC, "--cuda-device-only", "-S",
                                          "-o", asm, src],
                       check=True, capture_output=True)
        with open(asm) as f:
            return f.read()


def test_every_planned_shape_is_compiled(norm_asm):
    waits = _waits_between_streaming_loads(norm_asm)
    assert len(waits) == len(TYPES) * len(SHAPES), sorted(waits)


def test_no_full_wait_between_streaming_loads(norm_asm):
    waits = _waits_between_streaming_loads(norm_asm)
    bad = {k: v for k, v in waits.items() if v}
    assert not bad, "loads issued a round trip apart: %s" % bad


def test_checker_sees_a_serialized_load():
    """The counter itself: a wait between two streaming loads is counted, one after the last
    is not."""
    asm = "\n".join([
        "_ZN3arf14ar_norm_kernelIxEEvv:",
        "\tglobal_load_dwordx4 v[0:3], v0, s[0:1] nt",
        "\ts_waitcnt vmcnt(0)",
        "\tglobal_load_dwordx4 v[4:7], v0, s[2:3] nt",
        "\ts_waitcnt vmcnt(0)",
        "\ts_endpgm",
    ])
    assert _waits_between_streaming_loads(asm) == {"_ZN3arf14ar_norm_kernelIxEEvv": 1}
