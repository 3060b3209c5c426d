"""Pins of the oracle's stand-alone RMSNorm (host only): the normalisation step applied to a
stored tensor, which the unfused fallback computes in a second kernel.

Held to torch.nn.functional.rms_norm in float64 (an independent implementation), to closed forms
(constant row, one-hot row with eps = 0), to exact invariances (sign symmetry, power-of-two
scaling with eps scaled by 4^k), to the final rounding done by torch's casts, to odd row widths
(no vector alignment in the definition) and to the fused oracle: RMSNorm(residual_out) there
must equal this function applied to residual_out.
"""
import math

import numpy as np
import pytest
import torch

import synth

DTYPES = ["bf16", "fp16", "fp32"]
TD = synth.TORCH_DTYPES


def _values(a, dtype):
    if dtype == "fp32":
        return a.astype(np.float64)
    return torch.from_numpy(a.view(np.int16)).view(TD[dtype]).double().numpy()


def _store(values, dtype):
    t = torch.as_tensor(np.asarray(values, dtype=np.float64)).to(torch.float32).to(TD[dtype])
    return synth.storage_numpy(t)


def _x(M, H, dtype, seed, sigma=1.0):
    parts, _, gam = synth.custom(1, M, H, dtype, seed, dist=("normal", 0.0, sigma))
    return synth.storage_numpy(parts[0]), gam.numpy()


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("M,H,eps", [(3, 1, 1e-6), (2, 7, 1e-6), (4, 1001, 1e-5),
                                     (2, 7168, 1e-6), (1, 65544, 1e-6)])
def test_matches_torch_rms_norm_float64(oracle_mod, dtype, M, H, eps):
    x, gam = _x(M, H, dtype, 7 * H + M)
    out, y, rstd = oracle_mod.rmsnorm(x, gam, eps, dtype, debug=True)
    v = torch.from_numpy(_values(x, dtype))
    want = torch.nn.functional.rms_norm(v, (H,), weight=torch.from_numpy(gam).double(),
                                        eps=float(np.float32(eps)))
    np.testing.assert_allclose(y, want.numpy(), rtol=1e-12, atol=1e-300)
    assert np.array_equal(out, synth.storage_numpy(torch.from_numpy(y).to(torch.float32)
                                                   .to(TD[dtype])))
    ms = (_values(x, dtype) ** 2).mean(axis=1)
    np.testing.assert_allclose(rstd, 1.0 / np.sqrt(ms + float(np.float32(eps))), rtol=1e-12)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("c", [0.5, -3.0, 1.25])
def test_constant_row(oracle_mod, dtype, c):
    """x_i = c: y_i = c / sqrt(c^2 + eps) * gamma_i."""
    H, eps = 96, 1e-3
    x = _store(np.full((2, H), c), dtype)
    gam = np.linspace(0.5, 1.5, H).astype(np.float32)
    _, y, _ = oracle_mod.rmsnorm(x, gam, eps, dtype, debug=True)
    want = c / math.sqrt(c * c + float(np.float32(eps))) * gam.astype(np.float64)
    np.testing.assert_allclose(y, np.broadcast_to(want, (2, H)), rtol=1e-14)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("H,j,a", [(16, 3, 2.0), (1000, 999, -0.75), (5, 0, 8.0)])
def test_one_hot_row_eps_zero(oracle_mod, dtype, H, j, a):
    """x = a * e_j, eps = 0: y_j = sign(a) sqrt(H) gamma_j, every other y_i = 0."""
    v = np.zeros((1, H))
    v[0, j] = a
    x = _store(v, dtype)
    gam = np.linspace(0.75, 1.25, H).astype(np.float32)
    _, y, _ = oracle_mod.rmsnorm(x, gam, 0.0, dtype, debug=True)
    want = np.zeros((1, H))
    want[0, j] = math.copysign(math.sqrt(H), a) * float(gam[j])
    np.testing.assert_allclose(y, want, rtol=1e-14, atol=0)


@pytest.mark.parametrize("dtype", DTYPES)
def test_sign_symmetry(oracle_mod, dtype):
    x, gam = _x(3, 520, dtype, 5)
    neg = _store(-_values(x, dtype), dtype)
    out, y, _ = oracle_mod.rmsnorm(x, gam, 1e-6, dtype, debug=True)
    out_n, y_n, _ = oracle_mod.rmsnorm(neg, gam, 1e-6, dtype, debug=True)
    assert np.array_equal(y_n, -y)
    assert np.array_equal(_values(out_n, dtype), -_values(out, dtype))


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("k", [-3, 2])
def test_power_of_two_scale_invariance(oracle_mod, dtype, k):
    """x -> 2^k x with eps -> 4^k eps leaves y bit-identical (all steps scale exactly)."""
    x, gam = _x(2, 256, dtype, 11, sigma=0.5)
    xs = _store(_values(x, dtype) * 2.0 ** k, dtype)
    assert np.array_equal(_values(xs, dtype), _values(x, dtype) * 2.0 ** k)
    eps = 2.0 ** -20
    _, y, _ = oracle_mod.rmsnorm(x, gam, eps, dtype, debug=True)
    _, ys, _ = oracle_mod.rmsnorm(xs, gam, eps * 4.0 ** k, dtype, debug=True)
    assert np.array_equal(y, ys)


@pytest.mark.parametrize("dtype", DTYPES)
def test_equals_fused_oracle_norm_step(oracle_mod, dtype):
    """kARResidualRMSNorm's norm_out is RMSNorm of its own residual_out."""
    parts, res, gam = synth.custom(4, 5, 1016 if dtype != "fp32" else 1012, dtype, 3)
    parts = [synth.storage_numpy(p) for p in parts]
    ro, no, y, rstd = oracle_mod.ar_residual_rmsnorm(parts, synth.storage_numpy(res), gam.numpy(),
                                                     1e-6, dtype, debug=True)
    out, y2, rstd2 = oracle_mod.rmsnorm(ro, gam.numpy(), 1e-6, dtype, debug=True)
    assert np.array_equal(out, no)
    assert np.array_equal(y2, y) and np.array_equal(rstd2, rstd)


def test_rows_argument_and_rejects(oracle_mod):
    x, gam = _x(6, 64, "bf16", 1)
    full = oracle_mod.rmsnorm(x, gam, 1e-6, "bf16")
    part = np.zeros_like(full)
    oracle_mod.rmsnorm(x, gam, 1e-6, "bf16", rows=(2, 5), out=part)
    assert np.array_equal(part[2:5], full[2:5]) and not part[:2].any() and not part[5:].any()
    with pytest.raises(ValueError):
        oracle_mod.rmsnorm(x, gam, 1e-6, "bf16", rows=(4, 7))
    with pytest.raises(ValueError):
        oracle_mod.rmsnorm(x, gam[:10], 1e-6, "bf16")
