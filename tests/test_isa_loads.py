"""Code-generation check of the fused kernel's streaming loads (CPU only: hipcc cross-compiles the
gfx950 code to assembly, nothing runs).

The fused kernel is bandwidth-bound only if each thread has all loads of a rank batch in flight
together. The compiler's scheduler has twice turned an intended batch into one load per DRAM round
trip (`load, s_waitcnt vmcnt(0), load, ...`), correct but up to 2x slower, and tests that
compare results cannot see that. This test compiles the norm-kernel shapes the launch planner
picks for rows of whole vectors up to H = 8192 (one or two 16-byte vectors per thread with one
chain per batch: W <= 8, and W = 16 with one vector) for the three element types, and asserts
that no full wait (`s_waitcnt vmcnt(0)`) falls between two of a kernel's streaming loads; for
the wide-row shapes (4 or 8 vectors per thread, W >= 8) it allows waits between rank batches
but at most one per 4 loads, and the same bound holds for the split (workspace) kernel at
every W. The fixed rank batches (one, two or four ranks per batch) may wait between batches, at
most once per batch. For
the sum kernel it compiles every (W, vectors per thread) and checks its loop-free path (kernel
entry to the first store): whole rank batches only, with exactly one full wait between
consecutive batches and none inside one (16 loads per batch, 8 once a thread holds 32 or more
binary32 values).
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
# Wide rows (many vectors per thread, one or a few chains per batch): waits between rank batches
# are by design, but never one per load.
WIDE = [(8, 8), (16, 8), (32, 8), (64, 8), (16, 4), (64, 4)]
# Fixed rank batches (W, vectors per thread, ranks per batch; the planner's shapes from one row
# per CU on): a wait between rank batches is the point, a wait inside one is not.
RANK = ([(w, 2, 1) for w in (4, 8, 16)] + [(w, 4, 1) for w in (2, 4)] +
        [(w, 2, 2) for w in (4, 8, 16, 32, 64)] + [(w, 1, 2) for w in (32, 64)] + [(8, 2, 4)])
TYPES = ("Bf16", "F16", "F32")
TN = {"Bf16": "4Bf16", "F16": "3F16", "F32": "3F32"}


SUM_W = (1, 2, 4, 8, 16, 32, 64)
ROWS_K = (0, 1, 2, 4, 8)
SUM_U = (1, 2, 4)
KVEC = {"Bf16": 8, "F16": 8, "F32": 4}


def _source() -> str:
    refs = []
    for t in TYPES:
        for w, v in SHAPES + WIDE:
            refs.append("reinterpret_cast<const void*>(&arf::ar_norm_kernel<arf::%s, %d, %d, true>)"
                        % (t, w, v))
        for w, v, n in RANK:
            refs.append("reinterpret_cast<const void*>(&arf::ar_norm_kernel<arf::%s, %d, %d, true, "
                        "arf::StreamSource, false, %d>)" % (t, w, v, n))
        for w in SUM_W:
            for v in (1, 2):
                refs.append("reinterpret_cast<const void*>(&arf::ar_norm_split_kernel<arf::%s, %d, "
                            "%d, true>)" % (t, w, v))
            for u in SUM_U:
                refs.append("reinterpret_cast<const void*>(&arf::ar_sum_kernel<arf::%s, %d, %d, "
                            "true>)" % (t, w, u))
        for k in ROWS_K:
            refs.append("reinterpret_cast<const void*>(&arf::ar_rmsnorm_rows_kernel<arf::%s, %d>)"
                        % (t, k))
    return ('#include "ar_kernels.hpp"\n'
            "const void* const kKernels[] = {\n  " + ",\n  ".join(refs) + "};\n")


def _sum_batch_loads(W: int, U: int, kvec: int) -> int:
    """Streaming loads per rank batch of the sum kernel by design: ranks per batch x U, with 16
    loads per batch, 8 once a thread holds 32 or more binary32 values."""
    max_loads = 8 if U * kvec >= 32 else 16
    return max(1, min(max_loads // U, W)) * U


def _sum_fast_path_waits(asm: str) -> dict:
    """Per sum kernel symbol: (streaming loads, full waits between two of them) from the kernel
    entry to its first store (the loop-free path for a chunk wholly in range)."""
    out, name, done = {}, None, False
    for line in asm.splitlines():
        m = re.match(r"^(_Z\S*ar_sum_kernel\S*):", line)
        if m:
            name, done = m.group(1), False
            out[name] = [0, 0, False]
            continue
        if name is None or done:
            if "s_endpgm" in line:
                name = None
            continue
        r = out[name]
        if "global_store" in line:
            done = True
        elif "global_load" in line and " nt" in line:
            if r[2]:
                r[1] += 1
                r[2] = False
            r[0] += 1
        elif "s_waitcnt" in line and "vmcnt(0)" in line and r[0] > 0:
            r[2] = True
    return {k: (v[0], v[1]) for k, v in out.items()}


def _sum_symbol(t: str, w: int, u: int) -> str:
    tn = {"Bf16": "4Bf16", "F16": "3F16", "F32": "3F32"}[t]
    return "_ZN3arf13ar_sum_kernelINS_%sELi%dELi%dELb1ENS_12StreamSourceEEE" % (tn, w, u)


def _norm_symbol(t: str, w: int, v: int, ranks_per_batch: int = 0) -> str:
    return ("_ZN3arf14ar_norm_kernelINS_%sELi%dELi%dELb1ENS_12StreamSourceELb0ELi%dE"
            % (TN[t], w, v, ranks_per_batch))


def _norm_streaming_loads(asm: str, kernel: str = "ar_norm_kernel", stop: str = "") -> dict:
    """Per kernel symbol: its streaming (non-temporal) global loads (up to the first line that
    holds `stop`, if given)."""
    out, name = {}, None
    for line in asm.splitlines():
        m = re.match(r"^(_Z\S*%s\S*):" % kernel, line)
        if m:
            name = m.group(1)
            out[name] = 0
        elif name is not None and stop and stop in line:
            name = None
        elif name is not None and "global_load" in line and " nt" in line:
            out[name] += 1
        elif "s_endpgm" in line:
            name = None
    return out


def _waits_between_streaming_loads(asm: str, kernel: str = "ar_norm_kernel",
                                   stop: str = "") -> dict:
    """Per kernel symbol: the number of s_waitcnt vmcnt(0) that lie between two streaming
    (non-temporal) global loads of its body (up to the first line that holds `stop`)."""
    out, name, nt, pending = {}, None, 0, False
    for line in asm.splitlines():
        m = re.match(r"^(_Z\S*%s\S*):" % kernel, line)
        if m:
            name, nt, pending = m.group(1), 0, False
            out[name] = 0
            continue
        if name is None:
            continue
        if stop and stop in line:
            name = None
        elif "global_load" in line and " nt" in line:
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
    assert len(waits) == len(TYPES) * (len(SHAPES) + len(WIDE) + len(RANK)), sorted(waits)
    assert len(_sum_fast_path_waits(norm_asm)) == len(TYPES) * len(SUM_W) * len(SUM_U)


def test_sum_fast_path_waits_only_between_rank_batches(norm_asm):
    got = _sum_fast_path_waits(norm_asm)
    bad = []
    for t in TYPES:
        for w in SUM_W:
            for u in SUM_U:
                sym = [k for k in got if k.startswith(_sum_symbol(t, w, u))]
                assert len(sym) == 1, (t, w, u, sym)
                nt, waits = got[sym[0]]
                per_batch = _sum_batch_loads(w, u, KVEC[t])
                # Whole batches only, and one full wait between consecutive batches.
                if nt == 0 or nt % per_batch or waits != nt // per_batch - 1:
                    bad.append((t, w, u, nt, per_batch, waits))
    assert not bad, "(type, W, U, loads, loads per batch, full waits): %s" % bad


def test_no_full_wait_between_streaming_loads(norm_asm):
    waits = _waits_between_streaming_loads(norm_asm)
    narrow = [_norm_symbol(t, w, v) for t in TYPES for w, v in SHAPES]
    bad = {k: v for k, v in waits.items() if v and any(k.startswith(p) for p in narrow)}
    assert not bad, "loads issued a round trip apart: %s" % bad


def test_wide_rows_loads_not_serialized(norm_asm):
    """Wide-row shapes wait between rank batches, never after (nearly) every load: at most one
    full wait per 4 streaming loads (W = 16 with 8 vectors per thread once compiled to 135 waits
    for 136 loads, 1.6-4x slower)."""
    waits = _waits_between_streaming_loads(norm_asm)
    loads = _norm_streaming_loads(norm_asm)
    bad = []
    for t in TYPES:
        for w, v in WIDE:
            sym = [k for k in waits if k.startswith(_norm_symbol(t, w, v))]
            assert len(sym) == 1, (t, w, v, sym)
            if loads[sym[0]] == 0 or waits[sym[0]] * 4 > loads[sym[0]]:
                bad.append((t, w, v, loads[sym[0]], waits[sym[0]]))
    assert not bad, "(type, W, vectors per thread, loads, full waits): %s" % bad


def test_rank_batches_wait_only_between_batches(norm_asm):
    """Fixed rank batches: every streaming load of the unrolled chains is issued (the W + 1
    tensors' VPT vectors; the loop body of the 16-rank walk for W >= 32), and full waits number
    at most the rank batches (min(W, 16) / ranks per batch), never one per load of a batch."""
    waits = _waits_between_streaming_loads(norm_asm)
    loads = _norm_streaming_loads(norm_asm)
    bad = []
    for t in TYPES:
        for w, v, n in RANK:
            sym = [k for k in waits if k.startswith(_norm_symbol(t, w, v, n))]
            assert len(sym) == 1, (t, w, v, n, sym)
            ranks = min(w, 16)
            if loads[sym[0]] < (ranks + 1) * v or waits[sym[0]] > ranks // n:
                bad.append((t, w, v, n, loads[sym[0]], waits[sym[0]]))
    assert not bad, "(type, W, vectors per thread, ranks per batch, loads, full waits): %s" % bad


def _argument_rounds(asm: str, kernel: str) -> dict:
    """Per kernel symbol: the scalar-memory waits (`s_waitcnt lgkmcnt`) from the kernel's entry
    to its first streaming (non-temporal) load of the data, i.e. the dependent rounds of
    kernel-argument reads before the data is requested."""
    out, name = {}, None
    for line in asm.splitlines():
        m = re.match(r"^(_Z\S*%s\S*):" % kernel, line)
        if m:
            name = m.group(1)
            out[name] = 0
        elif name is not None:
            if re.search(r"\b(global|buffer)_load\S* .* nt", line):
                name = None
            elif "s_waitcnt" in line and "lgkmcnt" in line:
                out[name] += 1
            elif "s_endpgm" in line:
                name = None
    return out


def test_kernel_arguments_read_in_one_round(norm_asm):
    """Every kernel reads the arguments its first loads need in one round: one scalar wait before
    its first load of the data (two or three dependent rounds cost a decode-size call 2-3.5 %).
    Checked on the norm kernel's planned shapes, every sum and split kernel up to 16 ranks and
    the one-pass rows kernels, all three element types (the earlier form: 3 / 2 / 2 / 2)."""
    bad = []
    for kernel in ("ar_norm_kernel", "ar_sum_kernel", "ar_norm_split_kernel",
                   "ar_rmsnorm_rows_kernel"):
        rounds = _argument_rounds(norm_asm, kernel)
        assert rounds, kernel
        for sym, n in rounds.items():
            w = int(re.search(r"kernelINS_\w+?ELi(\d+)E", sym).group(1))
            # W > 16 ranks: the pointers stay with the 16-rank walk.  Rows kernel with K = 0
            # (rows past 8 vectors per thread): two passes over cached loads, no streaming one.
            if (kernel != "ar_rmsnorm_rows_kernel" and w > 16) or \
                    (kernel == "ar_rmsnorm_rows_kernel" and w == 0):
                continue
            if n != 1:
                bad.append((sym, n))
    assert not bad, "kernels reading their arguments in more than one round: %s" % bad


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


def test_split_kernel_loads_not_serialized(norm_asm):
    """The split (workspace) kernel, every W and one or two vectors per thread: at most one full
    wait per 4 streaming loads (it measured 1-3 waits for up to 68 loads) on its path to the
    first barrier (the segment's loads; what follows re-reads other segments only when a wait
    times out or the row's sum of squares leaves the binary32 range)."""
    waits = _waits_between_streaming_loads(norm_asm, "ar_norm_split_kernel", "s_barrier")
    loads = _norm_streaming_loads(norm_asm, "ar_norm_split_kernel", "s_barrier")
    assert len(waits) == len(TYPES) * len(SUM_W) * 2, sorted(waits)
    bad = {k: (loads[k], v) for k, v in waits.items() if loads[k] == 0 or v * 4 > loads[k]}
    assert not bad, "(loads, full waits): %s" % bad
