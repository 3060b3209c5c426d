"""Pins of the oracle's RMSNorm epilogue (host only).

The norm has no formula on the pages; the oracle uses textbook RMSNorm (Zhang & Sennrich 2019)
of the stored residual_out row.  These tests hold it to an independent library implementation
(torch.nn.functional.rms_norm in float64), to closed forms (unit RMS output, constant rows,
one-hot rows), to exact invariances (power-of-two scaling, sign symmetry) and to the final
rounding done by torch's casts.
"""
import math

import numpy as np
import pytest
import torch

import synth

DTYPES = ["bf16", "fp16", "fp32"]
TD = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}


def _values(a, dtype):
    if dtype == "fp32":
        return a.astype(np.float64)
    return torch.from_numpy(a.view(np.int16)).view(TD[dtype]).double().numpy()


def _store(values, dtype):
    t = torch.as_tensor(np.asarray(values, dtype=np.float64)).to(torch.float32).to(TD[dtype])
    return synth.storage_numpy(t)


def _inputs(W, M, H, dtype, seed, sigma=1.0):
    parts, res, gam = synth.custom(W, M, H, dtype, seed, dist=("normal", 0.0, sigma))
    return [synth.storage_numpy(p) for p in parts], synth.storage_numpy(res), gam.numpy()


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("W,M,H,eps", [(1, 3, 64, 1e-6), (2, 4, 256, 1e-6),
                                       (8, 5, 7168, 1e-6), (16, 2, 8192, 1e-5)])
def test_matches_torch_rms_norm_float64(oracle_mod, dtype, W, M, H, eps):
    """y == torch.nn.functional.rms_norm(residual_out, (H,), gamma, eps) in float64."""
    parts, res, gam = _inputs(W, M, H, dtype, 100 + W)
    ro, no, y, rstd = oracle_mod.ar_residual_rmsnorm(parts, res, gam, eps, dtype, debug=True)
    v = torch.from_numpy(_values(ro, dtype))
    want = torch.nn.functional.rms_norm(v, (H,), weight=torch.from_numpy(gam).double(),
                                        eps=float(np.float32(eps)))
    np.testing.assert_allclose(y, want.numpy(), rtol=1e-12, atol=1e-300)
    # norm_out is y rounded to binary32 and then to the storage type (torch casts).
    want_no = synth.storage_numpy(torch.from_numpy(y).to(torch.float32).to(TD[dtype]))
    assert np.array_equal(no, want_no)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("eps", [1e-6, 1e-5, 0.25])
def test_unit_rms_before_rounding(oracle_mod, dtype, eps):
    """With gamma = 1: sqrt(mean_i y_i^2) = sqrt(ms / (ms + eps)), ms = mean of squares."""
    parts, res, _ = _inputs(4, 6, 512, dtype, 21, sigma=0.3)
    gam = np.ones(512, dtype=np.float32)
    ro, _, y, rstd = oracle_mod.ar_residual_rmsnorm(parts, res, gam, eps, dtype, debug=True)
    v = _values(ro, dtype)
    ms = (v * v).mean(axis=1)
    e = float(np.float32(eps))
    np.testing.assert_allclose(np.sqrt((y * y).mean(axis=1)), np.sqrt(ms / (ms + e)),
                               rtol=1e-12)
    np.testing.assert_allclose(rstd, 1.0 / np.sqrt(ms + e), rtol=1e-14)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("c", [0.5, -3.0, 1.0 / 1024])
def test_constant_row(oracle_mod, dtype, c):
    """v_i == c: y_i = c / sqrt(c^2 + eps) * gamma_i."""
    H, eps = 128, 1e-6
    x0 = _store(np.full((2, H), c), dtype)
    zero = np.zeros_like(x0)
    gam = synth.custom(1, 1, H, dtype, 3)[2].numpy()
    _, _, y, _ = oracle_mod.ar_residual_rmsnorm([x0, zero], zero.copy(), gam, eps, dtype,
                                                debug=True)
    e = float(np.float32(eps))
    want = c / math.sqrt(c * c + e) * gam.astype(np.float64)
    np.testing.assert_allclose(y, np.broadcast_to(want, y.shape), rtol=1e-14)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("H,j,a", [(64, 0, 3.0), (7168, 5000, -0.25), (4096, 4095, 96.0)])
def test_one_hot_row_eps_zero(oracle_mod, dtype, H, j, a):
    """Only v_j = a != 0, eps = 0: y_j = sign(a) * sqrt(H) * gamma_j, all other y_i = 0."""
    x0 = np.zeros((1, H), dtype=np.float64)
    x0[0, j] = a
    x0 = _store(x0, dtype)
    zero = np.zeros_like(x0)
    gam = synth.custom(1, 1, H, dtype, 4)[2].numpy()
    _, _, y, _ = oracle_mod.ar_residual_rmsnorm([x0], zero, gam, 0.0, dtype, debug=True)
    want = np.zeros(H)
    want[j] = math.copysign(math.sqrt(H), a) * float(gam[j])
    np.testing.assert_allclose(y[0], want, rtol=1e-14, atol=0)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("k", [-3, 2, 5])
def test_power_of_two_scale_invariance(oracle_mod, dtype, k):
    """Scaling every input by 2^k and eps by 4^k leaves y bit-identical: every step of the norm
    scales exactly by a power of two."""
    parts, res, gam = _inputs(4, 4, 256, dtype, 31, sigma=0.5)
    eps = 2.0 ** -20
    _, _, y, _ = oracle_mod.ar_residual_rmsnorm(parts, res, gam, eps, dtype, debug=True)
    sc = 2.0 ** k
    parts2 = [_store(_values(p, dtype) * sc, dtype) for p in parts]
    res2 = _store(_values(res, dtype) * sc, dtype)
    _, _, y2, _ = oracle_mod.ar_residual_rmsnorm(parts2, res2, gam, eps * 4.0 ** k, dtype,
                                                 debug=True)
    assert np.array_equal(y, y2)


@pytest.mark.parametrize("dtype", DTYPES)
def test_sign_symmetry(oracle_mod, dtype):
    parts, res, gam = _inputs(8, 3, 384, dtype, 41)
    ro, no = oracle_mod.ar_residual_rmsnorm(parts, res, gam, 1e-6, dtype)
    if dtype == "fp32":
        flip = lambda a: (a.view(np.uint32) ^ np.uint32(1 << 31)).view(np.float32)
    else:
        flip = lambda a: a ^ np.uint16(0x8000)
    ro2, no2 = oracle_mod.ar_residual_rmsnorm([flip(p) for p in parts], flip(res), gam, 1e-6,
                                              dtype)
    assert np.array_equal(ro2, flip(ro))
    assert np.array_equal(no2, flip(no))


def test_gamma_scales_output(oracle_mod):
    """y is linear in gamma: doubling gamma doubles y exactly."""
    parts, res, gam = _inputs(2, 3, 256, "bf16", 51)
    _, _, y, _ = oracle_mod.ar_residual_rmsnorm(parts, res, gam, 1e-6, "bf16", debug=True)
    _, _, y2, _ = oracle_mod.ar_residual_rmsnorm(parts, res, gam * 2, 1e-6, "bf16", debug=True)
    assert np.array_equal(y * 2, y2)


def test_zero_row_with_zero_eps_is_nan(oracle_mod):
    """Degenerate row: all zeros with eps = 0 gives 0 * inf = NaN (IEEE)."""
    z = np.zeros((1, 16), dtype=np.uint16)
    _, no = oracle_mod.ar_residual_rmsnorm([z], z.copy(), np.ones(16, np.float32), 0.0, "bf16")
    assert ((no & 0x7F80) == 0x7F80).all() and ((no & 0x7F) != 0).all()


def test_norm_reads_rounded_residual_out(oracle_mod):
    """The norm reads the stored (rounded) residual_out: with bf16 partials 1 and 2^-9 the
    binary32 sum 1 + 2^-9 is stored as 1, so the row is constant 1 and, with eps = 0 and
    gamma = 1, y == 1 exactly."""
    H = 16
    one = _store(np.ones((1, H)), "bf16")
    tiny = _store(np.full((1, H), 2.0 ** -9), "bf16")
    zero = np.zeros_like(one)
    ro, no, y, _ = oracle_mod.ar_residual_rmsnorm([one, tiny], zero, np.ones(H, np.float32), 0.0,
                                                  "bf16", debug=True)
    assert (_values(ro, "bf16") == 1.0).all()
    assert (y == 1.0).all()
