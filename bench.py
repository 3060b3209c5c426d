#!/usr/bin/env python3
"""Benchmark of the fused all-reduce-sum + residual + RMSNorm core on one MI355X.

One step = one ar_residual_rmsnorm call (kARResidualRMSNorm: W partials summed in binary32,
residual added, residual_out and norm_out written) on the wide-hidden prefill workload:
W=8 partials, M=2048 tokens, H=7168, bf16.  Inputs are resident in HBM before the timed region.
Buffer sets are rotated so that the bytes a timed batch touches exceed the 256 MB Infinity
Cache (the numbers are HBM numbers, not cache numbers).  Steps are timed with HIP events on the
stream the kernel is launched on; events cut the timed steps into up to 5 windows, and the
headline is the median window's rate, with the windows' spread beside it.

Output: ONE JSON line with the metric (effective HBM GB/s = algorithmic bytes / time, bytes =
(W + 3) * M * H * 2: W partial reads, residual read, residual_out and norm_out writes), the
roofline of the kernel against the 8 TB/s HBM peak, the oracle's CPU baseline, and a sweep over
M = 1..2048 for both patterns (stream-launched and hipGraph-replayed µs/call).

Modes:
  (default)              the benchmark above
  --mode pmc             a short run for rocprofv3 --pmc: a plain device copy of known size
                         (calibrates FETCH_SIZE / WRITE_SIZE) and a few headline steps
  --summarize-stats DIR  markdown summary of a rocprofv3 --kernel-trace --stats output dir
  --summarize-pmc DIR... markdown summary of rocprofv3 --pmc output dirs (FETCH_SIZE run, then
                         WRITE_SIZE run) scaled by the copy calibration
  --summarize-sweep-trace DIR BENCH_JSON
                         per-M median in-kernel duration of the wide-hidden sweep kernels from a
                         rocprofv3 --kernel-trace dir, beside the per-call graph times of a
                         bench JSON line
  --phases               markdown table: where a decode-size call's time goes (the library's
                         kernels rebuilt with their phase hooks stamping a clock, beside the
                         same calls timed without them)
  --stream-counts        markdown table: the streaming probe's rate for 2 to 17 streams at the
                         headline's bytes per call
"""
from __future__ import annotations

import argparse
import csv
import ctypes
import glob
import hashlib
import json
import math
import os
import re
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E peak, GB/s
INFINITY_CACHE = 256 * 2 ** 20
ROTATE_BYTES = 512 * 2 ** 20   # bytes a timed batch must touch (2x the Infinity Cache)
COPY_CAL_BYTES = 256 * 2 ** 20

HEADLINE = dict(workload="wide_hidden", pattern="rms", W=8, M=2048, H=7168, dtype="bf16",
                eps=1e-6)
SWEEP_M = (1, 8, 32, 64, 128, 512, 2048)
PROFILE_DIR = os.path.join(ROOT, "profiles")
PMC_SUMMARY = os.path.join(PROFILE_DIR, "norm_kernel_wide_hidden_M2048_pmc.md")


def kernel_source_hash() -> str:
    """Hash of every source the library is built from (kernels, launch planning, build flags):
    counter figures taken on another build are not reported as this one's traffic."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "all_reduce_residual_amd", "csrc")
    paths = sorted(glob.glob(os.path.join(csrc, "*.hip")) + glob.glob(os.path.join(csrc, "*.hpp"))
                   + glob.glob(os.path.join(ROOT, "include", "*.h")))
    paths.append(os.path.join(ROOT, "all_reduce_residual_amd", "_build.py"))
    for path in paths:
        h.update(os.path.relpath(path, ROOT).encode())
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def metric_bytes(pattern: str, W: int, M: int, H: int, esize: int) -> int:
    """Algorithmic bytes of one call: W partials (+ residual) read, outputs written.  The
    two-kernel path is charged the fused op's bytes (same result, so the same metric); the
    stand-alone RMSNorm reads x and writes y."""
    if pattern == "rmsnorm":
        return 2 * M * H * esize
    extra = 3 if pattern in ("rms", "unfused", "rms_ws") else 1
    return (W + extra) * M * H * esize


# ---- GPU cases -------------------------------------------------------------------------------

def split_dims(M: int, S: int):
    """The split kernel's launch grid (blocks in x, y) for M rows of S segments: 8 x S with
    fewer than 8 rows (block (m, s); a row's segments on one XCD), S x M up to 65535 rows, else
    one dimension of M S blocks."""
    if M < 8:
        return 8, S
    return (S, M) if M <= 65535 else (M * S, 1)


class Case:
    """One (pattern, W, M, H) problem with R rotated buffer sets carved from one allocation per
    tensor role, and pre-marshalled C-ABI arguments for every set."""

    def __init__(self, ar, torch, pattern, W, M, H, dtype="bf16", eps=1e-6, rotate=True,
                 seed=1234, dist=(0.0, 0.05)):
        self.ar, self.torch = ar, torch
        self.pattern, self.W, self.M, self.H, self.dtype, self.eps = pattern, W, M, H, dtype, eps
        tdt = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[dtype]
        self.esize = 4 if dtype == "fp32" else 2
        self.bytes = metric_bytes(pattern, W, M, H, self.esize)
        footprint = self.bytes
        self.R = max(1, min(4096, math.ceil(ROTATE_BYTES / footprint))) if rotate else 1
        g = torch.Generator(device="cuda")
        g.manual_seed(seed)
        rows = self.R * M

        def randn(mu, sigma):
            t = torch.empty((rows, H), dtype=torch.float32, device="cuda")
            t.normal_(mu, sigma, generator=g)
            return t.to(tdt)

        self.parts = [randn(*dist) for _ in range(W)]
        if pattern in ("rms", "unfused", "rmsnorm", "rms_ws"):
            self.res = randn(0.0, 1.0)
            self.gamma = torch.empty(H, dtype=torch.float32, device="cuda").uniform_(
                0.8, 1.2, generator=g)
            self.ro = torch.empty_like(self.res)
            self.no = torch.empty_like(self.res)
            self.fn = {"rms": ar.lib().ar_residual_rmsnorm,
                       "unfused": ar.lib().ar_residual_rmsnorm_unfused,
                       "rmsnorm": ar.lib().ar_rmsnorm,
                       "rms_ws": ar.lib().ar_residual_rmsnorm_ws}[pattern]
            # One workspace serves every rotation set (calls on one stream never overlap).
            self.ws = ar.new_workspace(M, "cuda") if pattern == "rms_ws" else None
        else:
            self.out = torch.empty_like(self.parts[0])
            self.fn = ar.lib().ar_sum
        self.dt = ar.dtype_code(tdt)
        self._keep = []
        self.args = [self._args_for(r) for r in range(self.R)]
        torch.cuda.synchronize()

    def _sl(self, t, r):
        return t[r * self.M:(r + 1) * self.M].data_ptr()

    def _args_for(self, r):
        ptrs = (ctypes.c_void_p * self.W)(*[self._sl(p, r) for p in self.parts])
        self._keep.append(ptrs)
        if self.pattern == "rmsnorm":
            return (self._sl(self.res, r), self.M, self.H, self.dt, self.gamma.data_ptr(),
                    ctypes.c_float(self.eps), self._sl(self.no, r))
        if self.pattern in ("rms", "unfused", "rms_ws"):
            args = (ptrs, self.W, self.M, self.H, self.dt, self._sl(self.res, r),
                    self.gamma.data_ptr(), ctypes.c_float(self.eps), self._sl(self.ro, r),
                    self._sl(self.no, r))
            if self.pattern == "rms_ws":
                args += (self.ws.data_ptr(), self.ws.numel())
            return args
        return (ptrs, self.W, self.M, self.H, self.dt, self._sl(self.out, r))

    def call(self, i: int, stream_handle: int) -> None:
        st = self.fn(*self.args[i % self.R], ctypes.c_void_p(stream_handle))
        if st != 0:
            raise RuntimeError("library call failed: %s" % self.ar.status_string(st))

    def calls_per_batch(self, minimum: int) -> int:
        """A batch covers every rotation set equally and has at least `minimum` calls."""
        return self.R * max(1, math.ceil(minimum / self.R))

    def time_stream(self, calls: int, reps: int = 5) -> float:
        """Median µs/call of `calls` back-to-back launches on the current stream."""
        torch = self.torch
        s = torch.cuda.current_stream()
        h = s.cuda_stream
        for i in range(min(calls, 3 * self.R) + 3):
            self.call(i, h)
        torch.cuda.synchronize()
        res = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(s)
            for i in range(calls):
                self.call(i, h)
            b.record(s)
            b.synchronize()
            res.append(a.elapsed_time(b) * 1000.0 / calls)
        return sorted(res)[len(res) // 2]

    def time_graph(self, calls: int, reps: int = 5) -> float:
        """Median µs/call of a hipGraph replay holding `calls` launches.  The first `reps`
        replays are not timed: a newly built case ran its first replays up to 8 % slower
        (W = 8 H = 7168 M = 128: 6.69 against 6.2 µs), the next ones steadily."""
        torch = self.torch
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(3):
                self.call(i, side.cuda_stream)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            h = torch.cuda.current_stream().cuda_stream
            for i in range(calls):
                self.call(i, h)
        for _ in range(reps):
            graph.replay()
        torch.cuda.synchronize()
        res = []
        s = torch.cuda.current_stream()
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(s)
            graph.replay()
            b.record(s)
            b.synchronize()
            res.append(a.elapsed_time(b) * 1000.0 / calls)
        del graph
        return sorted(res)[len(res) // 2]


class GatherCase(Case):
    """All-gather share: W row slices of an [M, H] tensor gathered into it, R rotated sets."""

    def __init__(self, ar, torch, W, M, H, dtype="bf16"):
        self.ar, self.torch = ar, torch
        self.pattern, self.W, self.M, self.H, self.dtype = "gather", W, M, H, dtype
        tdt = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[dtype]
        self.esize = 4 if dtype == "fp32" else 2
        self.bytes = 2 * M * H * self.esize            # every slice read once, out written once
        self.R = max(1, min(4096, math.ceil(ROTATE_BYTES / self.bytes)))
        self.src = torch.empty((self.R * M, H), dtype=tdt, device="cuda").normal_()
        self.out = torch.empty_like(self.src)
        self.fn = ar.lib().ar_all_gather
        self.dt = ar.dtype_code(tdt)
        self._keep = []
        self.args = []
        for r in range(self.R):
            ptrs = []
            for j in range(W):
                b, c = ar.ar_row_partition(W, M, j)
                ptrs.append(self.src[r * M + b:r * M + b + c].data_ptr() if c else 0)
            arr = (ctypes.c_void_p * W)(*ptrs)
            self._keep.append(arr)
            self.args.append((arr, W, M, H, self.dt, self._sl(self.out, r)))
        torch.cuda.synchronize()


class LamportCase(Case):
    """Lamport-style one-shot exchange on one GPU: per round, W producer pushes (each writes its
    slot of this round's buffer and empties its slot of the next), then the polling consumer,
    which only reads.  `mode` "push" times the W pushes alone, "step" pushes + consumer (the
    three rotating buffers are the only set: the receive buffers are state, so small shapes are
    cache-warm), "consume" the consumer alone over the receive-buffer sets of prepare_consume,
    each holding a pushed round 0, in turn."""

    def __init__(self, ar, torch, pattern, W, M, H, dtype="bf16", eps=1e-6):
        self.ar, self.torch = ar, torch
        self.pattern, self.W, self.M, self.H, self.dtype, self.eps = pattern, W, M, H, dtype, eps
        tdt = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[dtype]
        self.esize = 4 if dtype == "fp32" else 2
        self.bytes = metric_bytes(pattern, W, M, H, self.esize)
        self.R = 1
        self.mode = "step"
        g = torch.Generator(device="cuda")
        g.manual_seed(99)
        self.parts = [torch.empty((M, H), dtype=torch.float32, device="cuda")
                      .normal_(0.0, 0.05, generator=g).to(tdt) for _ in range(W)]
        self.rbuf = torch.empty((ar.LAMPORT_BUFFERS, W, M, H), dtype=tdt, device="cuda")
        self.status = torch.zeros(1, dtype=torch.int32, device="cuda")
        self.dt = ar.dtype_code(tdt)
        L = ar.lib()
        self.L = L
        self.push_args = [(p.data_ptr(), r, self.rbuf.data_ptr(), W, M, H, self.dt)
                          for r, p in enumerate(self.parts)]
        if pattern == "rms":
            self.res = torch.empty((M, H), dtype=torch.float32, device="cuda").normal_(
                generator=g).to(tdt)
            self.gamma = torch.empty(H, dtype=torch.float32, device="cuda").uniform_(
                0.8, 1.2, generator=g)
            self.ro, self.no = torch.empty_like(self.res), torch.empty_like(self.res)
        else:
            self.out = torch.empty((M, H), dtype=tdt, device="cuda")
        self.sets = [self.rbuf]
        self._arm(self.rbuf)
        torch.cuda.synchronize()

    def _arm(self, rbuf) -> None:
        st = self.L.ar_lamport_arm(rbuf.data_ptr(), self.W, self.M, self.H, self.dt,
                                   ctypes.c_void_p(self.torch.cuda.current_stream().cuda_stream))
        if st != 0:
            raise RuntimeError("ar_lamport_arm failed: %s" % self.ar.status_string(st))

    def consume(self, rnd: int, h: int, rbuf=None) -> int:
        rb = (self.rbuf if rbuf is None else rbuf).data_ptr()
        W, M, H = self.W, self.M, self.H
        if self.pattern == "rms":
            return self.L.ar_lamport_residual_rmsnorm(
                rb, W, M, H, self.dt, rnd, self.res.data_ptr(), self.gamma.data_ptr(),
                ctypes.c_float(self.eps), self.ro.data_ptr(), self.no.data_ptr(),
                self.status.data_ptr(), 0, ctypes.c_void_p(h))
        return self.L.ar_lamport_sum(rb, W, M, H, self.dt, rnd, self.out.data_ptr(),
                                     self.status.data_ptr(), 0, ctypes.c_void_p(h))

    def prepare_consume(self) -> int:
        """Receive-buffer sets for "consume" mode, each armed and holding a pushed round 0:
        enough that one pass over them reads at least ROTATE_BYTES of slots (at most 64 sets), so
        the consumer's reads come from HBM as in the other timings.  Returns the set count."""
        torch = self.torch
        slot_bytes = self.W * self.M * self.H * self.esize        # the slots one round reads
        n = max(1, min(64, math.ceil(ROTATE_BYTES / slot_bytes)))
        self.sets = [self.rbuf] + [torch.empty_like(self.rbuf) for _ in range(n - 1)]
        h = torch.cuda.current_stream().cuda_stream
        for rb in self.sets:
            self._arm(rb)
            for r, p in enumerate(self.parts):
                st = self.L.ar_lamport_push(p.data_ptr(), r, rb.data_ptr(), self.W, self.M,
                                            self.H, self.dt, 0, ctypes.c_void_p(h))
                if st != 0:
                    raise RuntimeError("ar_lamport_push failed: %s" % self.ar.status_string(st))
        torch.cuda.synchronize()
        return n

    def call(self, i: int, stream_handle: int) -> None:
        """Round i: W pushes, then (in "step" mode) the consumer.  A graph holds a multiple of 3
        rounds, so that its replays keep the buffer rotation.  "consume" mode: the consumer of
        round 0 of set i mod (sets) alone (it only reads, so a pushed round can be consumed any
        number of times; its data is in place and no poll waits)."""
        if self.mode == "consume":
            st = self.consume(0, stream_handle, self.sets[i % len(self.sets)])
            if st != 0:
                raise RuntimeError("Lamport consumer failed: %s" % self.ar.status_string(st))
            return
        h = ctypes.c_void_p(stream_handle)
        for a in self.push_args:
            st = self.L.ar_lamport_push(*a, i, h)
            if st != 0:
                raise RuntimeError("ar_lamport_push failed: %s" % self.ar.status_string(st))
        if self.mode == "step":
            st = self.consume(i, stream_handle)
            if st != 0:
                raise RuntimeError("Lamport consumer failed: %s" % self.ar.status_string(st))


def headline_windows(steps: int, count: int = 5) -> list:
    """Step indices that cut `steps` timed steps into min(count, steps) windows of near-equal
    length: window j holds steps [b[j], b[j + 1])."""
    n = max(1, min(count, steps))
    return [(j * steps) // n for j in range(n + 1)]


def median(xs) -> float:
    v = sorted(xs)
    k = len(v) // 2
    return v[k] if len(v) % 2 else 0.5 * (v[k - 1] + v[k])


def lamport_lines(ar, torch, W=8, H=7168, Ms=(1, 8, 128, 512, 2048)) -> list:
    """hipGraph-replayed µs of the Lamport exchange: a round (W pushes + the consumer), the W
    pushes alone, and the consumer alone on a round already pushed (its data in place)."""
    lines = []
    for m in Ms:
        for pattern in ("rms", "sum"):
            c = LamportCase(ar, torch, pattern, W, m, H)
            calls = 21 if m >= 1024 else 99              # whole rotations of the 3 buffers
            c.mode = "step"
            us_step = c.time_graph(calls)
            c.mode = "push"
            us_push = c.time_graph(calls)
            c.mode = "step"
            us_step = min(us_step, c.time_graph(calls))
            sets = c.prepare_consume()
            c.mode = "consume"
            us_alone = c.time_graph(sets * max(1, math.ceil(calls / sets)))
            torch.cuda.synchronize()
            status = int(c.status.item())
            lines.append({"pattern": "kARResidualRMSNorm" if pattern == "rms" else "kAllReduce",
                          "W": W, "M": m, "H": H, "us_pushes": round(us_push, 3),
                          "us_step": round(us_step, 3),
                          "us_step_minus_pushes": round(us_step - us_push, 3),
                          "us_consumer_alone": round(us_alone, 3), "consume_sets": sets,
                          "consumer_GBs_metric": round(c.bytes / (us_alone * 1e-6) / 1e9, 1),
                          "status": status})
            print("# lamport %s" % json.dumps(lines[-1]), file=sys.stderr, flush=True)
            del c
            torch.cuda.empty_cache()
    return lines


class ProbeCase(Case):
    """The calibration probe (bench_probes/ar_probe.h): `nr` read streams and `nw` write streams of
    M x H bf16 each with no arithmetic that matters, R rotated sets."""

    def __init__(self, torch, L, nr, nw, M, H):
        self.torch, self.L, self.nr, self.nw = torch, L, nr, nw
        self.nvec = M * H * 2 // 16
        self.bytes = (nr + nw) * self.nvec * 16
        self.R = max(1, min(4096, math.ceil(ROTATE_BYTES / self.bytes)))
        n32 = self.R * self.nvec * 4
        self.ins = [torch.empty(n32, dtype=torch.int32, device="cuda").random_()
                    for _ in range(nr)]
        self.outs = [torch.empty(n32, dtype=torch.int32, device="cuda") for _ in range(2)]
        self._keep = []
        self.args = []
        for k in range(self.R):
            off = k * self.nvec * 16
            arr = (ctypes.c_void_p * nr)(*[t.data_ptr() + off for t in self.ins])
            self._keep.append(arr)
            self.args.append((arr, nr, nw, self.nvec, self.outs[0].data_ptr() + off,
                              self.outs[1].data_ptr() + off, 64))
        torch.cuda.synchronize()

    def call(self, i: int, stream_handle: int) -> None:
        if self.L.ar_probe_stream(*self.args[i % self.R], ctypes.c_void_p(stream_handle)) != 0:
            raise RuntimeError("ar_probe_stream failed")


def stream_ceiling(torch, H=None, Ms=(2048, 512)) -> list:
    """What the memory system delivers for the fused kernel's traffic (9 reads + 2 writes) and
    the sum's (8 + 1) at the headline sizes, with no arithmetic or row reduction in the way
    (hipGraph replay, rotated sets): the context for the kernels' fraction of 8 TB/s."""
    H = H or HEADLINE["H"]
    path = os.path.join(ROOT, "all_reduce_residual_amd", "libar_probe.so")
    if not os.path.exists(path):
        return [{"error": "calibration probe library not built"}]
    L = ctypes.CDLL(path)
    L.ar_probe_stream.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int64,
                                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                  ctypes.c_void_p]
    L.ar_probe_stream.restype = ctypes.c_int
    lines = []
    for m in Ms:
        for nr, nw in ((9, 2), (8, 1)):
            c = ProbeCase(torch, L, nr, nw, m, H)
            us = c.time_graph(c.calls_per_batch(60))
            gbs = c.bytes / (us * 1e-6) / 1e9
            lines.append({"streams": "%dR+%dW" % (nr, nw), "M": m, "H": H, "bytes": c.bytes,
                          "us_graph": round(us, 3), "GBs": round(gbs, 1),
                          "pct_of_peak": round(100 * gbs / HBM_PEAK_GBS, 2)})
            print("# ceiling %s" % json.dumps(lines[-1]), file=sys.stderr, flush=True)
            del c
            torch.cuda.empty_cache()
    return lines


def stream_count_table(torch, H=None) -> str:
    """How the memory system's rate depends on the number of streams (markdown): the probe with
    nr read and nw write streams, M chosen so that every line moves the headline's bytes
    ((W + 3) M H 2 at W = 8, M = 2048), hipGraph replay over rotated sets."""
    H = H or HEADLINE["H"]
    path = os.path.join(ROOT, "all_reduce_residual_amd", "libar_probe.so")
    if not os.path.exists(path):
        raise SystemExit("calibration probe library not built")
    L = ctypes.CDLL(path)
    L.ar_probe_stream.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int64,
                                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                  ctypes.c_void_p]
    L.ar_probe_stream.restype = ctypes.c_int
    total = metric_bytes("rms", HEADLINE["W"], HEADLINE["M"], H, 2)
    out = ["| streams | rows per stream | bytes per call | µs per call | GB/s | % of 8 TB/s |",
           "|---|---|---|---|---|---|"]
    for nr, nw in ((1, 1), (2, 1), (4, 1), (4, 2), (8, 1), (9, 2), (16, 1)):
        m = total // ((nr + nw) * H * 2)
        c = ProbeCase(torch, L, nr, nw, m, H)
        us = c.time_graph(c.calls_per_batch(60))
        gbs = c.bytes / (us * 1e-6) / 1e9
        out.append("| %dR+%dW | %d | %d | %.2f | %.0f | %.1f |" % (
            nr, nw, m, c.bytes, us, gbs, 100 * gbs / HBM_PEAK_GBS))
        print("# streams %s" % out[-1], file=sys.stderr, flush=True)
        del c
        torch.cuda.empty_cache()
    return "\n".join(out)


PHASE_NAMES = {
    0: ("loads done", "", "", "", ""),
    1: ("loads done", "rstd (row reduced)", "", "", ""),
    2: ("segment loaded", "segment sum of squares", "slot published", "all slots seen",
        "rstd"),
}


def phase_table(ar, torch) -> str:
    """Where the time of a decode-size call goes (markdown).  For each launch shape the library
    plans: µs per call of the library call itself (hipGraph replay, rotated sets, no stamps),
    then the same kernel rebuilt with its phase hooks storing the 100 MHz clock per block
    (ar_probe_phases): per call, the kernel span (first block's entry to the last block's last
    store issued), the gap from one kernel's last store issued to the next kernel's first
    block, and each phase's latest block, from the kernel's first entry."""
    path = os.path.join(ROOT, "all_reduce_residual_amd", "libar_probe.so")
    P = ctypes.CDLL(path)
    P.ar_probe_phases.argtypes = [ctypes.c_int] * 8 + [ctypes.POINTER(ctypes.c_double)]
    P.ar_probe_phases.restype = ctypes.c_int
    cases = []
    for W, H, Ms in ((8, 7168, (1, 8, 32, 128)), (2, 4096, (128,))):
        for M in Ms:
            cs = ar.ar_launch_config(ar.PATTERN_ALLREDUCE, W, M, H, ar.DTYPE_BF16)
            cn = ar.ar_launch_config(ar.PATTERN_AR_RESIDUAL_RMSNORM, W, M, H, ar.DTYPE_BF16)
            sp = ar.ar_split_config(W, M, H, ar.DTYPE_BF16)
            if W == 8 and M <= 32 and cs["vecs_per_thread"] in (1, 2):
                cases.append(("kAllReduce", "sum", 0, W, M, H, cs["threads_per_block"],
                              cs["vecs_per_thread"], cs["grid"], 0))
            if cn["rows_per_block"] == 1 and cn["vecs_per_thread"] in (1, 2):
                cases.append(("kARResidualRMSNorm, one block per row", "rms", 1, W, M, H,
                              cn["threads_per_block"], cn["vecs_per_thread"], cn["grid"], 0))
            if sp["segments"]:
                cases.append(("kARResidualRMSNorm, %d segments per row" % sp["segments"],
                              "rms_ws", 2, W, M, H, sp["threads_per_block"], 1,
                              split_dims(M, sp["segments"])[0] * split_dims(M, sp["segments"])[1],
                              sp["segments"]))
    cases.insert(0, ("empty kernel (launch floor)", None, 3, 8, 1, 7168, 64, 1, 1, 0))
    rows = ["| kernel | W | M | H | launch | per call, library (µs) | per call, stamped (µs) "
            "| span (µs) | gap (µs) | phases (µs after the first block's entry) |",
            "|---|---|---|---|---|---|---|---|---|---|"]
    for name, pat, kind, W, M, H, threads, vpt, grid, seg in cases:
        out = (ctypes.c_double * 11)()
        st = P.ar_probe_phases(kind, W, M, H, threads, vpt, grid, seg, out)
        if st != 0:
            raise RuntimeError("ar_probe_phases failed (%d) for %s W=%d M=%d" % (st, name, W, M))
        lib_us = None
        if pat is not None:
            c = Case(ar, torch, pat, W, M, H)
            lib_us = c.time_graph(c.calls_per_batch(200), reps=7)
            del c
            torch.cuda.empty_cache()
        names = PHASE_NAMES.get(kind, ())
        ph = ", ".join("%s %.2f" % (names[i], out[3 + i]) for i in range(len(names))
                       if names[i] and out[3 + i] >= 0)
        launch = "%d x %d thr x %d vec" % (grid, threads, vpt)
        rows.append("| %s | %d | %d | %d | %s | %s | %.2f | %.2f | %.2f | %s |" % (
            name, W, M, H, launch, "%.2f" % lib_us if lib_us is not None else "—", out[0],
            out[1], out[2], ph or "—"))
        print("# phases %s" % rows[-1], file=sys.stderr, flush=True)
    return "\n".join(rows)


def two_shot_lines(ar, torch, W=8, H=7168, Ms=(128, 512, 2048)) -> list:
    """One GPU's two-shot share: reduce-scatter of rank 0's row slice with the fused kernels,
    then the all-gather of each output (hipGraph replay, rotated buffers)."""
    lines = []
    for m in Ms:
        b, c = ar.ar_row_partition(W, m, 0)
        g = GatherCase(ar, torch, W, m, H)
        ag = g.time_graph(g.calls_per_batch(100))
        del g
        for pattern in ("rms", "sum"):
            rs = Case(ar, torch, pattern, W, c, H)
            us_rs = rs.time_graph(rs.calls_per_batch(100))
            n_out = 2 if pattern == "rms" else 1
            lines.append({"pattern": "kARResidualRMSNorm" if pattern == "rms" else "kAllReduce",
                          "M": m, "slice_rows": c, "us_reduce_scatter_share": round(us_rs, 3),
                          "us_all_gather_per_output": round(ag, 3),
                          "us_share_total": round(us_rs + n_out * ag, 3)})
            del rs
            torch.cuda.empty_cache()
            print("# two-shot %s" % json.dumps(lines[-1]), file=sys.stderr, flush=True)
    return lines


# The other workloads the metric is quoted on (configs besides the wide-hidden sweep), and the
# routing fallback: (label, pattern, W, M, H, dtype).
CONFIG_LINES = [
    ("tiny W=2 M=4 H=256", "rms", 2, 4, 256, "bf16"),
    ("Llama-3 decode W=2 M=128 H=4096", "rms", 2, 128, 4096, "bf16"),
    ("TP4 80 MiB W=4 M=5120 H=8192", "sum", 4, 5120, 8192, "bf16"),
    ("TP16 8 MiB fp16 W=16 M=512 H=8192", "rms", 16, 512, 8192, "fp16"),
    ("two-kernel path, W=8 M=2048 H=7168", "unfused", 8, 2048, 7168, "bf16"),
    ("two-kernel path, odd width W=8 M=2048 H=7170", "unfused", 8, 2048, 7170, "bf16"),
    ("stand-alone RMSNorm M=2048 H=7168", "rmsnorm", 1, 2048, 7168, "bf16"),
    ("stand-alone RMSNorm, odd width M=2048 H=7170", "rmsnorm", 1, 2048, 7170, "bf16"),
]


def config_lines(ar, torch) -> list:
    """hipGraph-replayed µs/call (rotated buffers) of CONFIG_LINES."""
    lines = []
    names = {"rms": "kARResidualRMSNorm", "sum": "kAllReduce",
             "unfused": "kARResidualRMSNorm (two kernels)", "rmsnorm": "RMSNorm"}
    for label, pattern, W, M, H, dt in CONFIG_LINES:
        c = Case(ar, torch, pattern, W, M, H, dtype=dt)
        us = c.time_graph(c.calls_per_batch(50 if c.bytes >= (64 << 20) else 200))
        gbs = c.bytes / (us * 1e-6) / 1e9
        lines.append({"config": label, "pattern": names[pattern], "W": W, "M": M, "H": H,
                      "element_type": dt, "bytes": c.bytes, "us_graph": round(us, 3),
                      "GBs": round(gbs, 1), "pct_of_peak": round(100 * gbs / HBM_PEAK_GBS, 2)})
        print("# config %s" % json.dumps(lines[-1]), file=sys.stderr, flush=True)
        del c
        torch.cuda.empty_cache()
    return lines


def headline_sample(torch, case) -> dict:
    """Put the seeded workload inputs into rotation set 0, run one call and keep host copies of
    sampled rows of its inputs and both outputs; the CPU leg compares them with the oracle."""
    import numpy as np
    import synth
    wl = synth.WORKLOADS[HEADLINE["workload"]]
    M = case.M
    parts, res, gam = synth.inputs(wl, M)
    for d, h in zip(case.parts, parts):
        d[:M].copy_(h)
    case.res[:M].copy_(res)
    case.gamma.copy_(gam)
    torch.cuda.synchronize()
    case.call(0, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    rows = sorted(set([0, 1, M // 2, M - 1] + [int(r) for r in rng.integers(0, M, size=12)]))
    return {"rows": rows, "eps": wl.eps, "dtype": wl.dtype,
            "parts": [synth.storage_numpy(p)[rows] for p in parts],
            "residual": synth.storage_numpy(res)[rows], "gamma": gam.numpy(),
            "residual_out": synth.storage_numpy(case.ro[:M].cpu())[rows],
            "norm_out": synth.storage_numpy(case.no[:M].cpu())[rows]}


def check_headline_parity(sample: dict) -> dict:
    """CPU leg: the sampled headline rows against the oracle run on those rows (residual_out
    bit-exact, norm_out within 1 ulp); raises on a mismatch."""
    import numpy as np
    import oracle
    ro, no = oracle.ar_residual_rmsnorm(sample["parts"], sample["residual"], sample["gamma"],
                                        sample["eps"], sample["dtype"])
    if not np.array_equal(sample["residual_out"], ro):
        raise AssertionError("bench parity: residual_out differs from the oracle")

    def ordered(b):
        b = b.astype(np.int32)
        return np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)

    worst = int(np.abs(ordered(sample["norm_out"]) - ordered(no)).max())
    if worst > 1:
        raise AssertionError("bench parity: norm_out %d ulp from the oracle" % worst)
    return {"rows_checked": len(sample["rows"]), "residual_out": "bit-exact",
            "norm_out_max_ulp": worst}


# ---- CPU baseline -------------------------------------------------------------------------------

def cpu_baseline(min_wall: float = 1.5) -> dict:
    """The oracle (unchanged) on the headline workload, row slices over the host's threads."""
    import oracle
    import synth
    wl = synth.WORKLOADS[HEADLINE["workload"]]
    M, H, W = HEADLINE["M"], HEADLINE["H"], HEADLINE["W"]
    parts, res, gam = synth.inputs(wl, M)
    hp = [synth.storage_numpy(p) for p in parts]
    hr = synth.storage_numpy(res)
    g = gam.numpy()
    import numpy as np
    ro = np.empty_like(hr)
    no = np.empty_like(hr)
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    threads = max(1, min(16, avail))
    bounds = [(M * i // threads, M * (i + 1) // threads) for i in range(threads)]

    def one_call():
        ts = [threading.Thread(target=oracle.ar_residual_rmsnorm,
                               args=(hp, hr, g, wl.eps, wl.dtype),
                               kwargs=dict(rows=b, residual_out=ro, norm_out=no))
              for b in bounds]
        for t in ts:
            t.start()
        for t in ts:
            t.join()

    one_call()  # warm-up
    n = 0
    t0 = time.perf_counter()
    while True:
        one_call()
        n += 1
        if time.perf_counter() - t0 >= min_wall:
            break
    dt = (time.perf_counter() - t0) / n
    nbytes = metric_bytes("rms", W, M, H, 2)
    # One-core figure on a 256-row slice.
    t1 = time.perf_counter()
    oracle.ar_residual_rmsnorm(hp, hr, g, wl.eps, wl.dtype, rows=(0, 256), residual_out=ro,
                               norm_out=no)
    dt1 = time.perf_counter() - t1
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": "full W=8 M=2048 H=7168 bf16 residual+RMSNorm call, rows split over %d "
                      "threads, %d call(s) timed (%.1f s wall, ~%.0f s CPU)" % (
                          threads, n, dt * n, dt * n * threads),
            "us_per_call": round(dt * 1e6, 1),
            "one_core_GBs": round(metric_bytes("rms", W, 256, H, 2) / dt1 / 1e9, 4),
            "cpu_model": cpu_model()}


def cpu_oracle_configs(min_wall: float = 0.3) -> list:
    """The oracle (unchanged) on the other workload configurations, one call at their full
    size (row slices over the host threads as for the headline's baseline; calls of fewer than
    2^20 input elements on one thread), repeated for at least `min_wall` seconds: milliseconds
    per call and GB/s of the same byte count."""
    import numpy as np

    import oracle
    import synth
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    threads = max(1, min(16, avail))
    out = []
    for name in ("tiny", "llama3_decode", "large_sum", "fp16_many_rank"):
        wl = synth.WORKLOADS[name]
        M = wl.Ms[0]
        parts, res, gam = synth.inputs(wl, M)
        hp = [synth.storage_numpy(p) for p in parts]
        pattern = "rms" if "rms" in wl.patterns else "sum"
        o1 = np.empty_like(hp[0])
        o2 = np.empty_like(hp[0])
        # Small calls on one thread: starting threads would cost more than the work.
        nt = 1 if (wl.W + 1) * M * wl.H < (1 << 20) else max(1, min(threads, M))
        bounds = [(M * i // nt, M * (i + 1) // nt) for i in range(nt)]
        if pattern == "rms":
            hr, g = synth.storage_numpy(res), gam.numpy()
            fn = lambda b: oracle.ar_residual_rmsnorm(hp, hr, g, wl.eps, wl.dtype, rows=b,  # noqa
                                                      residual_out=o1, norm_out=o2)
        else:
            fn = lambda b: oracle.ar_sum(hp, wl.dtype, rows=b, out=o1)  # noqa: E731

        def one_call():
            if nt == 1:
                fn(bounds[0])
                return
            ts = [threading.Thread(target=fn, args=(b,)) for b in bounds]
            for t in ts:
                t.start()
            for t in ts:
                t.join()

        one_call()
        n, t0 = 0, time.perf_counter()
        while True:
            one_call()
            n += 1
            if time.perf_counter() - t0 >= min_wall:
                break
        dt = (time.perf_counter() - t0) / n
        nbytes = metric_bytes(pattern, wl.W, M, wl.H, 4 if wl.dtype == "fp32" else 2)
        out.append({"config": name, "pattern": "kARResidualRMSNorm" if pattern == "rms"
                    else "kAllReduce", "W": wl.W, "M": M, "H": wl.H, "element_type": wl.dtype,
                    "threads": nt, "calls": n, "ms_per_call": round(dt * 1e3, 4),
                    "GBs": round(nbytes / dt / 1e9, 3)})
        print("# oracle %s" % json.dumps(out[-1]), file=sys.stderr, flush=True)
    return out


def box_facts(torch, ar) -> dict:
    """What the numbers were measured on: the GPU (name, architecture, compute units as the
    library's launch planning sees them, device memory) and the host (CPU model, threads this
    process may run on)."""
    props = torch.cuda.get_device_properties(0)
    return {"gpu": torch.cuda.get_device_name(0),
            "arch": getattr(props, "gcnArchName", "unknown"),
            "compute_units": ar.ar_device_cu_count(),
            "device_memory_GiB": round(props.total_memory / 2 ** 30, 1),
            "host_cpu": cpu_model(),
            "host_threads": len(os.sched_getaffinity(0))}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ---- rocprofv3 summaries ----------------------------------------------------------------------

def _read_csvs(d: str, pattern: str):
    rows = []
    for path in glob.glob(os.path.join(d, "**", pattern), recursive=True):
        with open(path) as f:
            rows.extend(csv.DictReader(f))
    return rows


def summarize_sweep_trace(d: str, bench_json: str) -> str:
    """In-kernel time (median kernel-trace duration) against the per-call hipGraph time for the
    wide-hidden sweep (W = 8, H = 7168 bf16): the difference is launch gap and ramp, not kernel."""
    rows = _read_csvs(d, "*kernel_trace.csv")
    if not rows:
        raise SystemExit("no kernel_trace.csv under %s" % d)
    with open(bench_json) as f:
        line = json.loads(f.read().strip().splitlines()[-1])
    per_call = {(e["pattern"], e["M"]): e for e in line.get("sweep", [])}
    for e in line.get("sweep", []):
        if "us_graph_workspace" in e:
            per_call[("kARResidualRMSNorm, split rows", e["M"])] = dict(
                e, us_graph=e["us_graph_workspace"])
    W, H = HEADLINE["W"], HEADLINE["H"]
    V = H // 8
    durs = {}
    for r in rows:
        name = r["Kernel_Name"]
        wg, grid = int(r["Workgroup_Size_X"]), int(r["Grid_Size_X"])
        sp = re.search(r"ar_norm_split_kernel<arf::Bf16, (\d+), (\d+), \w+>", name)
        if sp and int(sp.group(1)) == W:
            segments = -(-V // (wg * int(sp.group(2))))
            gy = int(r.get("Grid_Size_Y", 1) or 1)
            if grid // wg == 8 and gy == segments:     # fewer than 8 rows: the sweep's one such M
                few = [k[1] for k in per_call if k[0].endswith("split rows") and k[1] < 8]
                M = few[0] if len(few) == 1 else None
            else:
                M = gy if gy > 1 else grid // wg // segments
            durs.setdefault(("kARResidualRMSNorm, split rows", M), []).append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
            continue
        m = re.search(r"ar_(norm|sum)_kernel<arf::Bf16, (\d+), (\d+), \w+, arf::StreamSource", name)
        if not m or int(m.group(2)) != W:
            continue
        if m.group(1) == "norm":
            pattern, M = "kARResidualRMSNorm", grid // wg          # one row per block
        else:
            pattern, M = "kAllReduce", grid * int(m.group(3)) // V  # U vectors per thread
        durs.setdefault((pattern, M), []).append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    out = ["| pattern | M | metric bytes | dispatches | in-kernel µs (median) | in-kernel % of 8 TB/s |"
           " per-call µs (graph) | per-call % of 8 TB/s |", "|---|---|---|---|---|---|---|---|"]
    for key in sorted(durs, key=lambda k: (k[0], k[1])):
        if key not in per_call:
            continue
        e = per_call[key]
        ds = sorted(durs[key])
        med = ds[len(ds) // 2]
        out.append("| %s | %d | %d | %d | %.2f | %.1f | %.2f | %.1f |" % (
            key[0], key[1], e["bytes"], len(ds), med, 100 * e["bytes"] / (med * 1e3) / HBM_PEAK_GBS,
            e["us_graph"], 100 * e["bytes"] / (e["us_graph"] * 1e3) / HBM_PEAK_GBS))
    return "\n".join(out)


def summarize_stats(d: str) -> str:
    rows = _read_csvs(d, "*kernel_stats.csv")
    if not rows:
        raise SystemExit("no kernel_stats.csv under %s" % d)
    out = ["| kernel | calls | avg µs | min µs | max µs | share % |", "|---|---|---|---|---|---|"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        name = r["Name"].replace("(anonymous namespace)::", "")
        short = re.sub(r"\(.*", "", name)[:90]
        out.append("| `%s` | %s | %.2f | %.2f | %.2f | %.1f |" % (
            short, r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    return "\n".join(out)


def _pmc_by_kernel(d: str, counter: str):
    rows = _read_csvs(d, "*counter_collection.csv")
    vals = {}
    for r in rows:
        if r.get("Counter_Name") != counter:
            continue
        vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return vals


# The plain-sum workload whose counters the pmc mode also collects (80 MiB per partial).
PMC_SUM = {"W": 4, "M": 5120, "H": 8192}

# `--mode pmc --pmc-set kernels`: the other kernels' counter workloads.  Each entry: a name, the
# Case arguments, a pattern that picks its kernel out of the counter data, and the algorithmic
# bytes one dispatch reads and writes.
PMC_KERNELS = [
    dict(name="norm kernel, fp16 W=16 M=512 H=8192 (TP16 8 MiB)", pattern="rms", W=16, M=512,
         H=8192, dtype="fp16", kernel=r"ar_norm_kernel<arf::F16, 16, .*StreamSource",
         read=17 * 512 * 8192 * 2, write=2 * 512 * 8192 * 2),
    dict(name="split kernel, W=8 M=8 H=7168 bf16 (workspace form)", pattern="rms_ws", W=8, M=8,
         H=7168, dtype="bf16", kernel=r"ar_norm_split_kernel<arf::Bf16, 8,",
         read=9 * 8 * 7168 * 2, write=2 * 8 * 7168 * 2),
    dict(name="RMSNorm rows kernel, odd width M=2048 H=7170 bf16", pattern="rmsnorm", W=1,
         M=2048, H=7170, dtype="bf16", kernel=r"ar_rmsnorm_rows_kernel<arf::Bf16, 8",
         read=2048 * 7170 * 2, write=2048 * 7170 * 2),
    dict(name="Lamport fused consumer, W=8 M=2048 H=7168 bf16", pattern="lamport", W=8, M=2048,
         H=7168, dtype="bf16", kernel=r"ar_norm_kernel<arf::Bf16, 8, .*LamportSource",
         read=9 * 2048 * 7168 * 2, write=2 * 2048 * 7168 * 2),
    dict(name="Lamport push (one rank), W=8 M=2048 H=7168 bf16", pattern="lamport", W=8, M=2048,
         H=7168, dtype="bf16", kernel=r"ar_lamport_push_kernel<arf::Bf16>",
         read=2048 * 7168 * 2, write=2 * 2048 * 7168 * 2),
]


def summarize_pmc(fetch_dir: str, write_dir: str) -> str:
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of the norm kernel, scaled by what the same
    counters read for torch's device copy of COPY_CAL_BYTES (reads and writes that many bytes)."""
    fetch = _pmc_by_kernel(fetch_dir, "FETCH_SIZE")
    write = _pmc_by_kernel(write_dir, "WRITE_SIZE")

    def pick(d, pred):
        ks = [k for k in d if pred(k)]
        if not ks:
            raise SystemExit("kernel not found in counter data: %s" % list(d)[:5])
        vals = [v for k in ks for v in d[k]]
        return ks[0], sum(vals) / len(vals), len(vals)

    is_norm = lambda k: "ar_norm_kernel" in k
    is_copy = lambda k: k.startswith("__amd_rocclr_copyBuffer")   # hipMemcpy device-to-device
    kn, f_norm, n1 = pick(fetch, is_norm)
    kc, f_copy, n2 = pick(fetch, is_copy)
    _, w_norm, n3 = pick(write, is_norm)
    _, w_copy, n4 = pick(write, is_copy)
    f_factor = COPY_CAL_BYTES / (f_copy * 1024.0)
    w_factor = COPY_CAL_BYTES / (w_copy * 1024.0)
    W, M, H = HEADLINE["W"], HEADLINE["M"], HEADLINE["H"]
    alg_read = (W + 1) * M * H * 2
    alg_write = 2 * M * H * 2
    fetch_b = f_norm * 1024.0 * f_factor
    write_b = w_norm * 1024.0 * w_factor
    data = {"kernel_hash": kernel_source_hash(), "fetch_bytes": round(fetch_b),
            "write_bytes": round(write_b), "traffic_bytes": round(fetch_b + write_b),
            "algorithmic_read_bytes": alg_read, "algorithmic_write_bytes": alg_write,
            "fetch_factor": round(f_factor, 4), "write_factor": round(w_factor, 4)}
    lines = [
        "norm kernel: `%s` (%d + %d dispatches)" % (re.sub(r"\(.*", "", kn), n1, n3),
        "copy kernel: `%s` (%d + %d dispatches), %d bytes read and written per dispatch" % (
            re.sub(r"\(.*", "", kc)[:80], n2, n4, COPY_CAL_BYTES),
        "scale = copy bytes / (copy counter KiB * 1024); scaled bytes = norm counter KiB * 1024 "
        "* scale",
        "",
        "| counter | norm kernel KiB/dispatch | copy KiB/dispatch | scale | scaled bytes | "
        "algorithmic bytes | ratio |",
        "|---|---|---|---|---|---|---|",
        "| FETCH_SIZE | %.0f | %.0f | %.4f | %.0f | %d | %.3f |" % (
            f_norm, f_copy, f_factor, fetch_b, alg_read, fetch_b / alg_read),
        "| WRITE_SIZE | %.0f | %.0f | %.4f | %.0f | %d | %.3f |" % (
            w_norm, w_copy, w_factor, write_b, alg_write, write_b / alg_write),
        "",
        "traffic_json: " + json.dumps(data),
    ]
    # The plain sum on the 80 MiB payload, when the run holds it.
    sw = PMC_SUM
    is_sum = lambda k: re.search(r"ar_sum_kernel<arf::Bf16, %d, " % sw["W"], k) is not None
    if any(is_sum(k) for k in fetch) and any(is_sum(k) for k in write):
        ks, f_sum, m1 = pick(fetch, is_sum)
        _, w_sum, m2 = pick(write, is_sum)
        s_read = sw["W"] * sw["M"] * sw["H"] * 2
        s_write = sw["M"] * sw["H"] * 2
        sf, swb = f_sum * 1024.0 * f_factor, w_sum * 1024.0 * w_factor
        lines += [
            "",
            "sum kernel (W=%d, M=%d, H=%d bf16, 80 MiB per partial): `%s` (%d + %d dispatches)" % (
                sw["W"], sw["M"], sw["H"], re.sub(r"\(.*", "", ks), m1, m2),
            "",
            "| counter | sum kernel KiB/dispatch | scale | scaled bytes | algorithmic bytes | ratio |",
            "|---|---|---|---|---|---|",
            "| FETCH_SIZE | %.0f | %.4f | %.0f | %d | %.3f |" % (f_sum, f_factor, sf, s_read,
                                                            sf / s_read),
            "| WRITE_SIZE | %.0f | %.4f | %.0f | %d | %.3f |" % (w_sum, w_factor, swb, s_write,
                                                            swb / s_write),
        ]
    return "\n".join(lines)


def summarize_pmc_kernels(fetch_dir: str, write_dir: str) -> str:
    """The PMC_KERNELS table: per kernel, FETCH_SIZE / WRITE_SIZE per dispatch scaled by the copy
    calibration, against the algorithmic bytes."""
    fetch = _pmc_by_kernel(fetch_dir, "FETCH_SIZE")
    write = _pmc_by_kernel(write_dir, "WRITE_SIZE")

    def mean_of(d, pat):
        ks = [k for k in d if re.search(pat, k)]
        vals = [v for k in ks for v in d[k]]
        return (ks[0] if ks else None), (sum(vals) / len(vals) if vals else None), len(vals)

    _, f_copy, _ = mean_of(fetch, r"^__amd_rocclr_copyBuffer")
    _, w_copy, _ = mean_of(write, r"^__amd_rocclr_copyBuffer")
    if not f_copy or not w_copy:
        raise SystemExit("copy calibration kernel not found in counter data")
    f_factor = COPY_CAL_BYTES / (f_copy * 1024.0)
    w_factor = COPY_CAL_BYTES / (w_copy * 1024.0)
    lines = ["copy calibration: FETCH_SIZE scale %.4f, WRITE_SIZE scale %.4f (bytes per counter "
             "KiB * 1024)" % (f_factor, w_factor), "",
             "| kernel | dispatches | fetch bytes | algorithmic read | ratio | write bytes | "
             "algorithmic write | ratio |", "|---|---|---|---|---|---|---|---|"]
    for kc in PMC_KERNELS:
        kn, f, nf = mean_of(fetch, kc["kernel"])
        _, w, nw = mean_of(write, kc["kernel"])
        if kn is None or w is None:
            lines.append("| %s | not found | | | | | | |" % kc["name"])
            continue
        fb, wb = f * 1024.0 * f_factor, w * 1024.0 * w_factor
        lines.append("| %s (`%s`) | %d + %d | %.0f | %d | %.3f | %.0f | %d | %.3f |" % (
            kc["name"], re.sub(r"\(.*", "", kn)[:90], nf, nw, fb, kc["read"], fb / kc["read"],
            wb, kc["write"], wb / kc["write"]))
    lines += ["", "kernel_hash: " + kernel_source_hash()]
    return "\n".join(lines)


def read_traffic():
    """Traffic from the committed counter summary, if it was taken on the current kernel."""
    try:
        with open(PMC_SUMMARY) as f:
            for line in f:
                if line.startswith("traffic_json:"):
                    d = json.loads(line.split(":", 1)[1])
                    if d.get("kernel_hash") == kernel_source_hash():
                        return d["traffic_bytes"]
    except (OSError, ValueError):
        pass
    return None


# ---- main ---------------------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--mode", choices=["bench", "pmc"], default="bench")
    ap.add_argument("--pmc-set", choices=["headline", "kernels"], default="headline")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--summarize-stats", metavar="DIR")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--summarize-pmc-kernels", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--summarize-sweep-trace", nargs=2, metavar=("TRACE_DIR", "BENCH_JSON"))
    ap.add_argument("--phases", action="store_true")
    ap.add_argument("--stream-counts", action="store_true")
    args = ap.parse_args()

    if args.summarize_sweep_trace:
        print(summarize_sweep_trace(*args.summarize_sweep_trace))
        return 0
    if args.summarize_stats:
        print(summarize_stats(args.summarize_stats))
        return 0
    if args.summarize_pmc:
        print(summarize_pmc(*args.summarize_pmc))
        return 0
    if args.summarize_pmc_kernels:
        print(summarize_pmc_kernels(*args.summarize_pmc_kernels))
        return 0
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU's share of the fused all-reduce on a single MI355X and "
              "does not run on more than one GPU (got --gpus %d, WORLD_SIZE=%d)."
              % (args.gpus, world), file=sys.stderr)
        return 2

    import torch
    import all_reduce_residual_amd as ar
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    ar.lib()
    if args.phases:
        print(phase_table(ar, torch))
        return 0
    if args.stream_counts:
        print(stream_count_table(torch))
        return 0

    H, W, M = HEADLINE["H"], HEADLINE["W"], HEADLINE["M"]
    if args.mode == "pmc":
        # Copy calibration: torch's device copy reads and writes COPY_CAL_BYTES per dispatch.
        src = torch.empty(COPY_CAL_BYTES // 4, dtype=torch.float32, device="cuda").uniform_()
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        h = torch.cuda.current_stream().cuda_stream
        if args.pmc_set == "kernels":
            del src, dst
            done = set()
            for kc in PMC_KERNELS:
                key = (kc["pattern"], kc["W"], kc["M"], kc["H"], kc["dtype"])
                if key in done:
                    continue
                done.add(key)
                if kc["pattern"] == "lamport":
                    case = LamportCase(ar, torch, "rms", kc["W"], kc["M"], kc["H"], kc["dtype"])
                else:
                    case = Case(ar, torch, kc["pattern"], kc["W"], kc["M"], kc["H"],
                                dtype=kc["dtype"])
                for i in range(max(3, args.steps)):
                    case.call(i, h)
                torch.cuda.synchronize()
                print("# pmc %s: %d calls" % (kc["name"], max(3, args.steps)), file=sys.stderr,
                      flush=True)
                del case
                torch.cuda.empty_cache()
            print(json.dumps({"mode": "pmc", "set": "kernels", "copy_bytes": COPY_CAL_BYTES,
                              "calls": max(3, args.steps)}))
            return 0
        case = Case(ar, torch, "rms", W, M, H)
        for i in range(max(2, args.steps)):
            case.call(i, h)
        torch.cuda.synchronize()
        R = case.R
        del case
        torch.cuda.empty_cache()
        # The plain sum on the largest payload (W = 4 partials of 80 MiB), the same way.
        sw = PMC_SUM
        case = Case(ar, torch, "sum", sw["W"], sw["M"], sw["H"], dist=(0.0, 0.5))
        for i in range(max(2, args.steps)):
            case.call(i, h)
        torch.cuda.synchronize()
        print(json.dumps({"mode": "pmc", "copy_bytes": COPY_CAL_BYTES, "norm_calls":
                          max(2, args.steps), "rotation_sets": R, "sum_calls": max(2, args.steps),
                          "sum_rotation_sets": case.R}))
        return 0

    box = box_facts(torch, ar)
    print("# device: %s (%s), %d CUs, %.0f GiB, host %s, %d host threads" % (
        box["gpu"], box["arch"], box["compute_units"], box["device_memory_GiB"], box["host_cpu"],
        box["host_threads"]), file=sys.stderr, flush=True)

    # Headline: warm-up, then exactly `steps` timed steps on rotated buffer sets, split by
    # events into (up to) 5 windows of consecutive steps; the value is the median window's
    # rate and the spread of the windows is reported beside it.
    case = Case(ar, torch, "rms", W, M, H)
    sample = headline_sample(torch, case)
    s = torch.cuda.current_stream()
    hnd = s.cuda_stream
    for i in range(args.warmup):
        case.call(i, hnd)
    torch.cuda.synchronize()
    win = headline_windows(args.steps)
    ev = [torch.cuda.Event(enable_timing=True) for _ in win]
    ev[0].record(s)
    for j in range(1, len(win)):
        for i in range(win[j - 1], win[j]):
            case.call(i, hnd)
        ev[j].record(s)
    ev[-1].synchronize()
    torch.cuda.synchronize()
    ms_total = ev[0].elapsed_time(ev[-1])
    us_windows = [ev[j - 1].elapsed_time(ev[j]) * 1000.0 / (win[j] - win[j - 1])
                  for j in range(1, len(win))]
    us_per_call = median(us_windows)
    gbs = case.bytes / (us_per_call * 1e-6) / 1e9
    launch_cfg = ar.ar_launch_config(ar.PATTERN_AR_RESIDUAL_RMSNORM, W, M, H, ar.DTYPE_BF16)
    print("# headline: %.2f us/call, %.1f GB/s (%.1f%% of peak), R=%d sets, cfg=%s" % (
        us_per_call, gbs, 100 * gbs / HBM_PEAK_GBS, case.R, launch_cfg), file=sys.stderr,
        flush=True)
    del case
    torch.cuda.empty_cache()

    result = {
        "metric": "µs/call and effective HBM GB/s (% of peak), AR+residual+RMSNorm, W=8 H=7168",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_total / args.steps, 6),
        "us_per_call": round(us_per_call, 3),
        "windows": {"count": len(us_windows), "steps": [win[j] - win[j - 1]
                                                        for j in range(1, len(win))],
                    "us_per_call": [round(u, 3) for u in us_windows],
                    "median": round(us_per_call, 3), "min": round(min(us_windows), 3),
                    "max": round(max(us_windows), 3),
                    "spread_pct": round(100.0 * (max(us_windows) - min(us_windows)) /
                                        us_per_call, 2)},
        "pct_of_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "wide_hidden prefill, kARResidualRMSNorm", "W": W, "M": M,
                   "H": H, "element_type": "bf16", "gamma": "fp32", "eps": HEADLINE["eps"],
                   "bytes_per_call": metric_bytes("rms", W, M, H, 2),
                   "launch": launch_cfg, "parity": None},
    }
    result["box"] = box
    traffic = read_traffic()
    result["roofline"] = {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                          "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                          "traffic": traffic}

    # Calibrations: minimal-work launch floor and device-copy bandwidth.
    floor = Case(ar, torch, "sum", 1, 1, 8, rotate=False)
    calib = {"launch_floor_us_stream": round(floor.time_stream(200), 3),
             "launch_floor_us_graph": round(floor.time_graph(200), 3)}
    del floor
    src = torch.empty(2 ** 30 // 4, dtype=torch.float32, device="cuda").uniform_()
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    ts = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        e1.synchronize()
        ts.append(e0.elapsed_time(e1))
    calib["d2d_copy_GBs"] = round(2 * 2 ** 30 / (sorted(ts)[2] * 1e-3) / 1e9, 1)
    del src, dst
    torch.cuda.empty_cache()
    calib["stream_ceiling"] = stream_ceiling(torch)
    result["calibration"] = calib

    if not args.no_sweep:
        sweep = []
        for pattern in ("rms", "sum"):
            for m in SWEEP_M:
                c = Case(ar, torch, pattern, W, m, H)
                calls = c.calls_per_batch(50 if m >= 512 else 200)
                us_s = c.time_stream(calls)
                us_g = c.time_graph(calls)
                warm = Case(ar, torch, pattern, W, m, H, rotate=False) if c.R > 1 else c
                us_w = warm.time_graph(200)
                best = min(us_s, us_g)
                sweep.append({"pattern": "kARResidualRMSNorm" if pattern == "rms" else
                              "kAllReduce", "M": m, "bytes": c.bytes, "rotation_sets": c.R,
                              "us_stream": round(us_s, 3), "us_graph": round(us_g, 3),
                              "us_graph_cache_warm": round(us_w, 3),
                              "GBs": round(c.bytes / (best * 1e-6) / 1e9, 1),
                              "pct_of_peak": round(100 * c.bytes / (best * 1e-6) / 1e9 /
                                                   HBM_PEAK_GBS, 2)})
                if pattern == "rms":
                    # The workspace form: rows split over several blocks where the heuristic
                    # splits them (ar_split_config), else the same kernel as above.
                    seg = ar.ar_split_config(W, m, H, ar.DTYPE_BF16)["segments"]
                    if seg:
                        cw = Case(ar, torch, "rms_ws", W, m, H)
                        us_ws = cw.time_graph(cw.calls_per_batch(200))
                        sweep[-1].update({"split_segments": seg,
                                          "us_graph_workspace": round(us_ws, 3)})
                        del cw
                print("# sweep %s" % json.dumps(sweep[-1]), file=sys.stderr, flush=True)
                del c, warm
                torch.cuda.empty_cache()
        result["sweep"] = sweep
        result["two_shot_share"] = two_shot_lines(ar, torch)
        result["configs"] = config_lines(ar, torch)
        result["lamport_exchange"] = lamport_lines(ar, torch)

    if not args.no_cpu:
        # The CPU leg: the oracle timed on the host cores, and the headline's sampled rows
        # checked against it.
        result["cpu_baseline"] = cpu_baseline()
        result["cpu_baseline"]["other_configs"] = cpu_oracle_configs()
        result["config"]["parity"] = check_headline_parity(sample)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
