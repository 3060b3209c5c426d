"""Parity of the two-kernel (unfused) kARResidualRMSNorm path and of the stand-alone RMSNorm
with the oracle (GPU, through the C ABI).

The two-kernel path is the routing fallback for norm rows the fused kernel does not take (odd
widths, rows wider than the register-resident limit).  Bar as for the fused path: residual_out
bit-identical, norm_out within 1 ulp (16-bit) or 1e-5 relative (binary32).  Also checked: the
two-kernel path agrees with the fused kernel where both apply, in-place calls, special values
and the full wide-hidden prefill shape on sampled rows.
"""
import numpy as np
import pytest
import torch

import all_reduce_residual_amd as ar
import synth
from gpu_util import assert_bit_exact, assert_norm_close, dev, host_np

pytestmark = pytest.mark.gpu

TD = synth.TORCH_DTYPES


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    ar.lib()


def _unfused(parts, res, gam, eps):
    d_parts = [dev(p) for p in parts]
    d_res, d_gam = dev(res), dev(gam)
    ro, no = torch.empty_like(d_res), torch.empty_like(d_res)
    ar.ar_residual_rmsnorm_unfused(d_parts, d_res, d_gam, eps, ro, no)
    torch.cuda.synchronize()
    return host_np(ro.cpu()), host_np(no.cpu())


def _check_unfused(oracle_mod, parts, res, gam, eps, dtype):
    ro, no = _unfused(parts, res, gam, eps)
    want_ro, want_no = oracle_mod.ar_residual_rmsnorm([host_np(p) for p in parts], host_np(res),
                                                      gam.numpy(), eps, dtype)
    assert_bit_exact(ro, want_ro, dtype, "residual_out")
    assert_norm_close(no, want_no, dtype)


# Odd widths (not whole 16-byte vectors), rows past the fused limit, and ordinary rows.
SHAPES = [(3, 1), (2, 7), (5, 13), (4, 1001), (3, 7170), (2, 65544), (1, 131072), (7, 7168),
          (33, 4096), (2, 8)]


@pytest.mark.parametrize("M,H", SHAPES, ids=["M%d-H%d" % s for s in SHAPES])
@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_unfused_matches_oracle(oracle_mod, M, H, dtype):
    print("case unfused", M, H, dtype, flush=True)
    parts, res, gam = synth.custom(4, M, H, dtype, seed=17 * H + M)
    _check_unfused(oracle_mod, parts, res, gam, 1e-6, dtype)


@pytest.mark.parametrize("W", [1, 2, 8, 16, 32, 64])
def test_unfused_world_sizes(oracle_mod, W):
    parts, res, gam = synth.custom(W, 3, 1020 + 2, "bf16", seed=W)
    _check_unfused(oracle_mod, parts, res, gam, 1e-5, "bf16")


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_unfused_agrees_with_fused(dtype):
    """Where both paths apply: residual_out identical, norm_out within the norm bar."""
    H = 7168 if dtype != "fp32" else 4096
    parts, res, gam = synth.custom(8, 37, H, dtype, seed=5)
    d_parts = [dev(p) for p in parts]
    d_res, d_gam = dev(res), dev(gam)
    ro1, no1 = torch.empty_like(d_res), torch.empty_like(d_res)
    ro2, no2 = torch.empty_like(d_res), torch.empty_like(d_res)
    ar.ar_residual_rmsnorm(d_parts, d_res, d_gam, 1e-6, ro1, no1)
    ar.ar_residual_rmsnorm_unfused(d_parts, d_res, d_gam, 1e-6, ro2, no2)
    torch.cuda.synchronize()
    assert_bit_exact(host_np(ro2.cpu()), host_np(ro1.cpu()), dtype, "residual_out")
    assert_norm_close(host_np(no2.cpu()), host_np(no1.cpu()), dtype)


def test_unfused_in_place_residual(oracle_mod):
    """residual_out may be the residual buffer itself."""
    dtype, M, H = "bf16", 6, 7170
    parts, res, gam = synth.custom(4, M, H, dtype, seed=9)
    want_ro, want_no = oracle_mod.ar_residual_rmsnorm([host_np(p) for p in parts], host_np(res),
                                                      gam.numpy(), 1e-6, dtype)
    d_parts = [dev(p) for p in parts]
    d_res = dev(res)
    no = torch.empty_like(d_res)
    ar.ar_residual_rmsnorm_unfused(d_parts, d_res, dev(gam), 1e-6, d_res, no)
    torch.cuda.synchronize()
    assert_bit_exact(host_np(d_res.cpu()), want_ro, dtype, "residual_out")
    assert_norm_close(host_np(no.cpu()), want_no, dtype)


def test_unfused_wide_hidden_prefill_sampled(oracle_mod):
    """W = 8, M = 2048, H = 7168 bf16 (the prefill shape) through the two-kernel path; the
    oracle checks 64 sampled rows."""
    wl = synth.WORKLOADS["wide_hidden"]
    parts, res, gam = synth.inputs(wl, 2048)
    d_parts = [dev(p) for p in parts]
    d_res = dev(res)
    ro, no = torch.empty_like(d_res), torch.empty_like(d_res)
    ar.ar_residual_rmsnorm_unfused(d_parts, d_res, dev(gam), wl.eps, ro, no)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    rows = sorted(set(rng.integers(0, 2048, 62).tolist()) | {0, 2047})
    h_parts = [host_np(p) for p in parts]
    h_ro, h_no = host_np(ro.cpu()), host_np(no.cpu())
    for r in rows:
        want_ro, want_no = oracle_mod.ar_residual_rmsnorm([p[r:r + 1] for p in h_parts],
                                                          host_np(res)[r:r + 1], gam.numpy(),
                                                          wl.eps, "bf16")
        assert_bit_exact(h_ro[r:r + 1], want_ro, "bf16", "residual_out row %d" % r)
        assert_norm_close(h_no[r:r + 1], want_no, "bf16", "norm_out row %d" % r)


def test_unfused_zero_rows():
    x = torch.empty(0, 7, dtype=torch.bfloat16, device="cuda")
    g = torch.ones(7, dtype=torch.float32, device="cuda")
    ar.ar_residual_rmsnorm_unfused([x, x], x, g, 1e-6, torch.empty_like(x), torch.empty_like(x))
    ar.ar_rmsnorm(x, g, 1e-6, torch.empty_like(x))


# ---- stand-alone RMSNorm ---------------------------------------------------------------------------

# Odd widths reach every vectors-per-thread choice of the any-width kernel (1, 2, 4, 8 and the
# two-pass form): 1001, 7170, 12345, 40001, 65544 / 200003 at 16 bits.
RMS_SHAPES = [(1, 1), (4, 7), (3, 64), (9, 256), (5, 1001), (17, 7168), (2, 8192), (3, 65536),
              (2, 65544), (1, 200003), (300, 128), (3, 7170), (3, 12345), (2, 40001),
              (600, 13)]


@pytest.mark.parametrize("M,H", RMS_SHAPES, ids=["M%d-H%d" % s for s in RMS_SHAPES])
@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_rmsnorm_matches_oracle(oracle_mod, M, H, dtype):
    print("case rmsnorm", M, H, dtype, flush=True)
    parts, _, gam = synth.custom(1, M, H, dtype, seed=3 * H + M)
    x = dev(parts[0])
    y = torch.empty_like(x)
    ar.ar_rmsnorm(x, dev(gam), 1e-6, y)
    torch.cuda.synchronize()
    want = oracle_mod.rmsnorm(host_np(parts[0]), gam.numpy(), 1e-6, dtype)
    assert_norm_close(host_np(y.cpu()), want, dtype)


# Odd widths in the row kernel's planned shapes at many rows (8 or more per CU: blocks of at most
# 192 threads, 128 with 8 vectors per thread) and at few rows (at most one per CU: the widest
# block up to 1024 threads; two per CU: up to 704); one case runs in place.
ROW_PLAN = [(2048, 7170, "bf16", False), (2048, 2562, "fp16", False), (2048, 1539, "fp32", False),
            (4096, 3074, "bf16", False), (8, 16386, "bf16", False), (64, 5122, "fp32", False),
            (1, 7170, "fp16", False), (100, 6146, "bf16", False), (2048, 7170, "fp16", True),
            (512, 8194, "bf16", False), (384, 16386, "bf16", False), (500, 5122, "fp32", False),
            (2048, 16386, "bf16", False), (1024, 9002, "fp32", False), (800, 20002, "fp16", True)]


@pytest.mark.parametrize("M,H,dtype,in_place", ROW_PLAN,
                         ids=["M%d-H%d-%s%s" % (m, h, d, "-inplace" if i else "")
                              for m, h, d, i in ROW_PLAN])
def test_rmsnorm_planned_row_shapes(oracle_mod, M, H, dtype, in_place):
    print("case rmsnorm rows", M, H, dtype, in_place, flush=True)
    parts, _, gam = synth.custom(1, M, H, dtype, seed=5 * H + M)
    x = dev(parts[0])
    y = x if in_place else torch.empty_like(x)
    ar.ar_rmsnorm(x, dev(gam), 1e-6, y)
    torch.cuda.synchronize()
    want = oracle_mod.rmsnorm(host_np(parts[0]), gam.numpy(), 1e-6, dtype)
    assert_norm_close(host_np(y.cpu()), want, dtype)

@pytest.mark.parametrize("H", [7168, 1001, 40001, 70001])
def test_rmsnorm_in_place(oracle_mod, H):
    parts, _, gam = synth.custom(1, 6, H, "fp16", seed=H)
    want = oracle_mod.rmsnorm(host_np(parts[0]), gam.numpy(), 1e-5, "fp16")
    x = dev(parts[0])
    ar.ar_rmsnorm(x, dev(gam), 1e-5, x)
    torch.cuda.synchronize()
    assert_norm_close(host_np(x.cpu()), want, "fp16")


@pytest.mark.parametrize("H", [256, 13])
@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_rmsnorm_special_values(oracle_mod, H, dtype):
    """Rows holding infinities, NaN, subnormals, zeros and the largest finite values, on both
    kernels (H = 256 is whole vectors, H = 13 is not).  Row 1 holds no infinity or NaN, so its
    finite values up to the largest of the type overflow a binary32 sum of squares (the oracle's
    is binary64); row 2 holds only subnormals and zeros."""
    rng = np.random.default_rng(H)
    if dtype == "fp32":
        pool = np.array([0.0, -0.0, 1e-45, 3.0, -2.5, np.inf, np.nan, 1e15, 3.4028235e38,
                         -1e30], dtype=np.float32)
        finite = pool[np.isfinite(pool)]
        x = torch.from_numpy(rng.choice(pool, size=(6, H)).astype(np.float32))
        x[1] = torch.from_numpy(rng.choice(finite, size=H).astype(np.float32))
        x[2] = torch.from_numpy(rng.choice(np.array([0.0, 1e-45, -3e-45, 1e-40], dtype=np.float32),
                                           size=H))
    else:
        pool = ([0x0000, 0x8000, 0x0001, 0x3C00, 0xC100, 0x7C00, 0x7E00, 0x7BFF] if dtype == "fp16"
                else [0x0000, 0x8000, 0x0001, 0x3F80, 0xC020, 0x7F80, 0x7FC0, 0x5A00, 0x7F7F,
                      0xF0A0])
        finite = [b for b in pool if (b & 0x7C00) != 0x7C00] if dtype == "fp16" else \
            [b for b in pool if (b & 0x7F80) != 0x7F80]
        sub = [0x0000, 0x0001, 0x8003, 0x0040] if dtype == "bf16" else [0x0000, 0x0001, 0x8003]
        xs = rng.choice(np.array(pool, dtype=np.uint16), size=(6, H))
        xs[1] = rng.choice(np.array(finite, dtype=np.uint16), size=H)
        xs[2] = rng.choice(np.array(sub, dtype=np.uint16), size=H)
        x = torch.from_numpy(xs.view(np.int16)).view(TD[dtype])
    x[0] = 1  # one ordinary row
    gam = torch.ones(H, dtype=torch.float32)
    d = dev(x)
    for eps in (1e-6, 0.0):
        y = torch.empty_like(d)
        ar.ar_rmsnorm(d, dev(gam), eps, y)
        torch.cuda.synchronize()
        want = oracle_mod.rmsnorm(host_np(x), gam.numpy(), eps, dtype)
        assert_norm_close(host_np(y.cpu()), want, dtype, "norm_out eps=%g" % eps)


# The residual sum at sizes its launch plan covers with one resident round of 256-thread blocks
# (W + 1 <= 8 operands: one vector per thread), whole rows and odd widths with an element tail.
ROUND = [(1, 128, 7168), (2, 128, 7168), (4, 128, 7168), (2, 100, 7170), (4, 57, 7169)]


@pytest.mark.parametrize("W,M,H", ROUND, ids=["W%d-M%d-H%d" % c for c in ROUND])
def test_unfused_resident_round_sizes(oracle_mod, W, M, H):
    print("case unfused", W, M, H, flush=True)
    parts, res, gam = synth.custom(W, M, H, "bf16", seed=W * 7 + M + H)
    _check_unfused(oracle_mod, parts, res, gam, 1e-6, "bf16")
