"""Rows whose sum of squares leaves the binary32 range, through every norm entry point.

The kernels reduce a row's sum of squares in binary32; the oracle in binary64.  Finite rows with
an RMS from about 1.8e19 / sqrt(H) up (or single elements above about 1.8e19) overflow that sum,
and rows far below 2^-63 with eps = 0 underflow it.  The kernels detect such rows and normalise
them again from the same rounded values scaled by a power of two; these tests compare the result
with the oracle at the usual bar (residual_out bit-identical, norm_out within 1 ulp for 16-bit
types and 1e-5 relative for binary32), with in-range rows in the same call, the same wave
(narrow rows) and the same block (several multi-wave rows per block) as the out-of-range ones.

Row recipe (per row: a magnitude s; every partial and the residual N(0, 1) * s, so residual_out
has an RMS of about s sqrt(W + 1)): s in {1, 1e18, 1e20, 1e25, 1e30, 1e35, 1e37}, a row whose
element 5 is the largest finite value of T (partial 0 holds it, every other addend is 0 there),
and a row of largest finite values; with eps = 0: s in {1, 2^-70, 2^-90, 2^-110, 2^-126, 2^-130}
and a row of zeros except one tiny element.
"""
import numpy as np
import pytest
import torch

import all_reduce_residual_amd as ar
import synth
from gpu_util import assert_bit_exact, assert_norm_close, dev, host_np

pytestmark = pytest.mark.gpu

TD = synth.TORCH_DTYPES
FMAX = {"bf16": float(torch.finfo(torch.bfloat16).max), "fp32": float(np.finfo(np.float32).max),
        "fp16": float(np.finfo(np.float16).max)}
BIG = [1.0, 1e18, 1e20, 1e25, 1e30, 1e35, 1e37]
TINY = [1.0, 2.0 ** -70, 2.0 ** -90, 2.0 ** -110, 2.0 ** -126, 2.0 ** -130]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    ar.lib()


def range_inputs(W, H, dtype, kind, seed, rows_per_scale=1):
    """Partials, residual and gamma whose residual_out rows span the binary32 edge (see the
    module docstring).  kind: "big" (eps > 0 rows of large magnitude) or "tiny" (eps = 0 rows
    of small magnitude)."""
    g = torch.Generator().manual_seed(seed)
    scales = BIG if kind == "big" else TINY
    rows = [s for s in scales for _ in range(rows_per_scale)]
    M = len(rows) + (2 if kind == "big" else 1)
    addends = []
    for _ in range(W + 1):
        x = torch.randn((M, H), generator=g, dtype=torch.float64)
        for i, s in enumerate(rows):
            x[i] *= s
        addends.append(x)
    fmax = FMAX[dtype]
    if kind == "big":
        # Row M-2: one element at the largest finite value; row M-1: all of them.
        for j, x in enumerate(addends):
            x[M - 2, 5] = fmax if j == 0 else 0.0
            x[M - 1] = fmax if j == 0 else 0.0
    else:
        # Row M-1: zeros but one element of the smallest normal magnitude of binary32 / 4.
        for j, x in enumerate(addends):
            x[M - 1] = 0.0
            if j == 0:
                x[M - 1, 3] = 2.0 ** -128
    parts = [x.to(torch.float32).to(TD[dtype]) for x in addends[:W]]
    res = addends[W].to(torch.float32).to(TD[dtype])
    gam = (torch.rand((H,), generator=g, dtype=torch.float32) + 0.5)
    eps = 1e-6 if kind == "big" else 0.0
    return parts, res, gam, eps


def want_rms(oracle_mod, parts, res, gam, eps, dtype):
    return oracle_mod.ar_residual_rmsnorm([host_np(p) for p in parts], host_np(res), gam.numpy(),
                                          eps, dtype)


def check(got_ro, got_no, want, dtype):
    assert_bit_exact(host_np(got_ro.cpu()), want[0], dtype, "residual_out")
    assert_norm_close(host_np(got_no.cpu()), want[1], dtype)


def _out_of_range_rows_exist(want_ro, dtype, eps):
    """Sanity: the inputs do reach the edge (some row's binary32 sum of squares overflows or, with
    eps = 0, underflows)."""
    x = want_ro.astype(np.float32) if dtype == "fp32" else (
        (want_ro.astype(np.uint32) << 16).view(np.float32) if dtype == "bf16" else
        want_ro.view(np.float16).astype(np.float32))
    with np.errstate(over="ignore", under="ignore"):
        ss = (x.astype(np.float32) ** 2).sum(axis=1, dtype=np.float32)
    return bool((~np.isfinite(ss)).any() or (eps == 0.0 and (ss < 2.0 ** -90).any()))


CASES = [(dt, kind, H) for dt in ("bf16", "fp32") for kind in ("big", "tiny")
         for H in (256, 1024, 7168)]


@pytest.mark.parametrize("dtype,kind,H", CASES, ids=["%s-%s-H%d" % c for c in CASES])
def test_fused_planned(oracle_mod, dtype, kind, H):
    """ar_residual_rmsnorm in its planned shape: H = 256 puts two rows in one wave (a row of 32
    or 64 lanes), H = 1024 / 7168 one multi-wave row per block."""
    print("case fused", dtype, kind, H, flush=True)
    parts, res, gam, eps = range_inputs(4, H, dtype, kind, seed=H + len(kind))
    want = want_rms(oracle_mod, parts, res, gam, eps, dtype)
    assert _out_of_range_rows_exist(want[0], dtype, eps)
    d_parts, d_res = [dev(p) for p in parts], dev(res)
    ro, no = torch.empty_like(d_res), torch.empty_like(d_res)
    ar.ar_residual_rmsnorm(d_parts, d_res, dev(gam), eps, ro, no)
    torch.cuda.synchronize()
    check(ro, no, want, dtype)


# Several multi-wave rows per block (2 or 4 rows of 128 or 512 lanes), several narrow rows per
# wave, with in-range and out-of-range rows mixed in one block: (type, H, threads, vectors per
# thread, lanes per row).
SHAPED = [("bf16", 1024, 256, 1, 128), ("bf16", 1024, 512, 1, 128), ("fp32", 1024, 256, 2, 128),
          ("bf16", 256, 256, 1, 32), ("fp32", 256, 64, 1, 64), ("bf16", 7168, 1024, 2, 512)]


@pytest.mark.parametrize("kind", ["big", "tiny"])
@pytest.mark.parametrize("dtype,H,threads,vpt,lanes", SHAPED,
                         ids=["%s-H%d-t%d-v%d-l%d" % c for c in SHAPED])
def test_fused_explicit_shapes(oracle_mod, kind, dtype, H, threads, vpt, lanes):
    print("case shaped", kind, dtype, H, threads, vpt, lanes, flush=True)
    vec = 4 if dtype == "fp32" else 8
    assert lanes * vpt * vec >= H and threads % lanes == 0
    parts, res, gam, eps = range_inputs(2, H, dtype, kind, seed=threads + lanes + vpt)
    want = want_rms(oracle_mod, parts, res, gam, eps, dtype)
    M = res.shape[0]
    rows = threads // lanes
    cfg = {"threads_per_block": threads, "vecs_per_thread": vpt, "lanes_per_row": lanes,
           "rows_per_block": rows, "grid": (M + rows - 1) // rows, "flat": 0, "nt_store": 1}
    d_parts, d_res = [dev(p) for p in parts], dev(res)
    ro, no = torch.empty_like(d_res), torch.empty_like(d_res)
    ar.ar_residual_rmsnorm(d_parts, d_res, dev(gam), eps, ro, no, config=cfg)
    torch.cuda.synchronize()
    check(ro, no, want, dtype)


@pytest.mark.parametrize("kind", ["big", "tiny"])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_fused_grid_stride(oracle_mod, kind, dtype):
    """A grid of 2 blocks walking all row groups: the out-of-range path inside the row loop,
    followed by in-range rows in the same block."""
    H = 1024
    parts, res, gam, eps = range_inputs(2, H, dtype, kind, seed=7, rows_per_scale=3)
    want = want_rms(oracle_mod, parts, res, gam, eps, dtype)
    vec = 4 if dtype == "fp32" else 8
    cfg = {"threads_per_block": 256, "vecs_per_thread": 1 if dtype == "bf16" else 2,
           "lanes_per_row": 128, "rows_per_block": 2, "grid": 2, "flat": 0, "nt_store": 0}
    assert cfg["lanes_per_row"] * cfg["vecs_per_thread"] * vec >= H
    d_parts, d_res = [dev(p) for p in parts], dev(res)
    ro, no = torch.empty_like(d_res), torch.empty_like(d_res)
    ar.ar_residual_rmsnorm(d_parts, d_res, dev(gam), eps, ro, no, config=cfg)
    torch.cuda.synchronize()
    check(ro, no, want, dtype)


@pytest.mark.parametrize("kind", ["big", "tiny"])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_split_rows(oracle_mod, kind, dtype):
    """ar_residual_rmsnorm_ws on a few-row shape the planner splits (W = 8, H = 7168), the split
    kernel with an explicit shape of 4 segments, and the same shape with no polls at all (every
    block computes every segment's sum itself before the range branch)."""
    W, H = 8, 7168
    parts, res, gam, eps = range_inputs(W, H, dtype, kind, seed=11)
    M = res.shape[0]
    dcode = ar.DTYPE_FP32 if dtype == "fp32" else ar.DTYPE_BF16
    assert ar.ar_split_config(W, M, H, dcode)["segments"] > 1
    want = want_rms(oracle_mod, parts, res, gam, eps, dtype)
    d_parts, d_res, d_gam = [dev(p) for p in parts], dev(res), dev(gam)
    ws = ar.new_workspace(M, "cuda")
    seg4 = -(-(H * (4 if dtype == "fp32" else 2) // 16) // 256)
    for cfg in (None,
                {"threads_per_block": 256, "vecs_per_thread": 1, "segments": seg4,
                 "max_polls": 1 << 14},
                {"threads_per_block": 256, "vecs_per_thread": 1, "segments": seg4,
                 "max_polls": 0}):
        print("case split", kind, dtype, cfg, flush=True)
        ro, no = torch.empty_like(d_res), torch.empty_like(d_res)
        ar.ar_residual_rmsnorm_ws(d_parts, d_res, d_gam, eps, ro, no, ws, config=cfg)
        torch.cuda.synchronize()
        check(ro, no, want, dtype)


@pytest.mark.parametrize("kind", ["big", "tiny"])
@pytest.mark.parametrize("dtype,H", [("bf16", 1024), ("fp32", 1024), ("bf16", 1030),
                                     ("fp32", 1027), ("bf16", 70001)])
def test_rmsnorm_and_two_kernel_path(oracle_mod, kind, dtype, H):
    """ar_rmsnorm (whole vectors: the fused kernel's norm-only mode; odd widths: the row kernel
    with values in registers; H = 70001: its two-pass form) and the two-kernel path."""
    print("case rmsnorm", kind, dtype, H, flush=True)
    parts, res, gam, eps = range_inputs(2, H, dtype, kind, seed=H)
    want = want_rms(oracle_mod, parts, res, gam, eps, dtype)
    d_parts, d_res, d_gam = [dev(p) for p in parts], dev(res), dev(gam)
    ro, no = torch.empty_like(d_res), torch.empty_like(d_res)
    ar.ar_residual_rmsnorm_unfused(d_parts, d_res, d_gam, eps, ro, no)
    torch.cuda.synchronize()
    check(ro, no, want, dtype)
    # The normalisation alone, of the stored residual_out, out of place and in place.
    want_y = oracle_mod.rmsnorm(want[0], gam.numpy(), eps, dtype)
    y = torch.empty_like(ro)
    ar.ar_rmsnorm(ro, d_gam, eps, y)
    ar.ar_rmsnorm(ro, d_gam, eps, ro)
    torch.cuda.synchronize()
    assert_norm_close(host_np(y.cpu()), want_y, dtype)
    assert_norm_close(host_np(ro.cpu()), want_y, dtype, "in place")


@pytest.mark.parametrize("kind", ["big", "tiny"])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_lamport_consumer(oracle_mod, kind, dtype):
    W, H = 4, 1024
    parts, res, gam, eps = range_inputs(W, H, dtype, kind, seed=5)
    want = want_rms(oracle_mod, parts, res, gam, eps, dtype)
    M = res.shape[0]
    d_parts, d_res = [dev(p) for p in parts], dev(res)
    rbuf = torch.empty((ar.LAMPORT_BUFFERS, W, M, H), dtype=TD[dtype], device="cuda")
    ar.ar_lamport_arm(rbuf)
    for r, p in enumerate(d_parts):
        ar.ar_lamport_push(p, r, rbuf, 0)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    ro, no = torch.empty_like(d_res), torch.empty_like(d_res)
    ar.ar_lamport_residual_rmsnorm(rbuf, 0, d_res, dev(gam), eps, ro, no, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    check(ro, no, want, dtype)


def test_fp16_never_leaves_the_range(oracle_mod):
    """binary16 cannot reach the edge (65504^2 * 65536 < 2^128; the smallest subnormal squared is
    2^-48): the largest fp16 rows and eps = 0 tiny rows stay on the binary32 path and match."""
    for kind in ("big", "tiny"):
        parts, res, gam, eps = range_inputs(2, 1024, "fp16", kind, seed=3)
        want = want_rms(oracle_mod, parts, res, gam, eps, "fp16")
        d_parts, d_res = [dev(p) for p in parts], dev(res)
        ro, no = torch.empty_like(d_res), torch.empty_like(d_res)
        ar.ar_residual_rmsnorm(d_parts, d_res, dev(gam), eps, ro, no)
        torch.cuda.synchronize()
        check(ro, no, want, "fp16")
