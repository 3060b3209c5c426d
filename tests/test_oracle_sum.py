"""Pins of the oracle's rank sum (kAllReduce) and residual add (host only).

Each test targets a mistake the oracle could plausibly make (a dropped or repeated rank, a wrong
index or transposed operand, rounding per step in the narrow type instead of one binary32 chain,
a different summation order, lost signed zeros) with something other than the oracle itself:
exact integer arithmetic, closed forms, an exact-rational replay with independently written
rounding, symmetry, and the recursive-summation error bound.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import synth
from exact_arith import from_bits, round_nearest_even, to_bits

DTYPES = ["bf16", "fp16", "fp32"]
NP_STORAGE = {"bf16": np.uint16, "fp16": np.uint16, "fp32": np.float32}
TD = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}


def _store(values, dtype):
    """binary32/64 values -> storage array via torch's round-to-nearest-even cast."""
    t = torch.as_tensor(np.asarray(values, dtype=np.float64)).to(torch.float32).to(TD[dtype])
    return synth.storage_numpy(t)


def _values(a, dtype):
    t = torch.from_numpy(a.view(np.int16) if dtype != "fp32" else a)
    if dtype != "fp32":
        t = t.view(TD[dtype])
    return t.double().numpy()


def _rand_inputs(W, M, H, dtype, seed, scale=1.0):
    parts, res, gam = synth.custom(W, M, H, dtype, seed, dist=("normal", 0.0, scale))
    return ([synth.storage_numpy(p) for p in parts], synth.storage_numpy(res), gam.numpy())


@pytest.mark.parametrize("dtype", DTYPES)
def test_single_rank_is_identity(oracle_mod, dtype):
    parts, _, _ = _rand_inputs(1, 5, 24, dtype, 1)
    x = parts[0].copy()
    # Include signed zeros, subnormals of the type and extremes.
    flat = x.reshape(-1)
    specials = {"bf16": [0x8000, 0x0000, 0x0001, 0x807F, 0x7F7F, 0xFF7F],
                "fp16": [0x8000, 0x0000, 0x0001, 0x83FF, 0x7BFF, 0xFBFF],
                "fp32": None}[dtype]
    if specials:
        flat[:len(specials)] = specials
    else:
        flat[:4] = np.array([-0.0, 1e-45, -3.4028235e38, 1.17549435e-38], dtype=np.float32)
    out = oracle_mod.ar_sum([x], dtype)
    assert out.view(np.uint16 if dtype != "fp32" else np.uint32).tolist() == \
        x.view(np.uint16 if dtype != "fp32" else np.uint32).tolist()


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("W", [2, 3, 8, 16, 64])
def test_integer_partials_exact(oracle_mod, dtype, W):
    """Integer-valued partials: every partial sum is an integer below 2^24, so the binary32
    chain is exact and the result is RN_T(exact integer sum).  The expected value is computed
    with Python/numpy integers, and each element's value encodes (rank, row, column), so a
    dropped rank, a repeated rank or a transposed index changes the sum."""
    M, H = 3, 40
    r = np.arange(W)[:, None, None]
    m = np.arange(M)[None, :, None]
    i = np.arange(H)[None, None, :]
    ints = ((r * 7 + 1) * (m * 3 + 2) + i * (r + 1)) % 251 - 125      # |v| <= 125, exact in T
    ints = np.where((r + m + i) % 5 == 0, -ints, ints)
    parts = [_store(ints[k], dtype) for k in range(W)]
    assert np.array_equal(_values(parts[0], dtype), ints[0])   # inputs are exact
    out = oracle_mod.ar_sum(parts, dtype)
    want = _store(ints.sum(axis=0), dtype)
    assert np.array_equal(out, want)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("W,c", [(2, 0.75), (8, 0.375), (16, -1.5), (64, 0.0078125), (4, 3.0)])
def test_constant_partials_closed_form(oracle_mod, dtype, W, c):
    """x_r == c for every rank: out = RN_T(W * c) (dyadic c, so every partial sum is exact)."""
    parts = [_store(np.full((2, 16), c), dtype) for _ in range(W)]
    out = oracle_mod.ar_sum(parts, dtype)
    assert np.array_equal(_values(out, dtype), np.full((2, 16), W * c))


def test_fixed_rank_order_binary32_chain(oracle_mod):
    """2^24 + 1 + 1 in binary32: the rank-order chain rounds 2^24 + 1 to 2^24 (tie to even)
    twice and yields 2^24; any other grouping ((1 + 1) + 2^24) yields 2^24 + 2."""
    x0 = np.full((1, 4), 2.0 ** 24, dtype=np.float32)
    x1 = np.ones((1, 4), dtype=np.float32)
    out = oracle_mod.ar_sum([x0, x1, x1.copy()], "fp32")
    assert (out == 2.0 ** 24).all()
    out = oracle_mod.ar_sum([x1, x1.copy(), x0], "fp32")
    assert (out == 2.0 ** 24 + 2).all()


def test_one_rounding_to_storage_type(oracle_mod):
    """1 + 2^-8 + 2^-8 with bf16 partials: binary32 accumulates exactly to 1 + 2^-7, which is a
    bf16 value; rounding to bf16 after every add would give 1 (two ties to even)."""
    parts = [_store(np.full((1, 8), v), "bf16") for v in (1.0, 2.0 ** -8, 2.0 ** -8)]
    out = oracle_mod.ar_sum(parts, "bf16")
    assert (_values(out, "bf16") == 1.0 + 2.0 ** -7).all()


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_negative_zero_seed(oracle_mod, dtype):
    """Seeding the chain with x_0 keeps -0 when every addend is -0 (a +0 seed would not)."""
    nz = np.full((1, 8), 0x8000, dtype=np.uint16)
    out = oracle_mod.ar_sum([nz, nz.copy(), nz.copy()], dtype)
    assert (out == 0x8000).all()


@pytest.mark.parametrize("dtype", DTYPES)
def test_sign_symmetry(oracle_mod, dtype):
    parts, _, _ = _rand_inputs(8, 6, 64, dtype, 7)
    out = oracle_mod.ar_sum(parts, dtype)
    if dtype == "fp32":
        neg = [-p for p in parts]
        out_n = oracle_mod.ar_sum(neg, dtype)
        assert np.array_equal(out_n.view(np.uint32), (out.view(np.uint32) ^ np.uint32(1 << 31)))
    else:
        neg = [p ^ np.uint16(0x8000) for p in parts]
        out_n = oracle_mod.ar_sum(neg, dtype)
        assert np.array_equal(out_n, out ^ np.uint16(0x8000))


@pytest.mark.parametrize("dtype", DTYPES)
def test_appending_zero_ranks(oracle_mod, dtype):
    parts, _, _ = _rand_inputs(4, 6, 64, dtype, 9)
    zero = np.zeros_like(parts[0])
    out = oracle_mod.ar_sum(parts, dtype)
    out_z = oracle_mod.ar_sum(parts + [zero, zero.copy(), zero.copy(), zero.copy()], dtype)
    # x + (+0) == x for every x except -0 (-0 + +0 = +0); drop -0 results from the comparison.
    if dtype == "fp32":
        keep = out.view(np.uint32) != 0x80000000
    else:
        keep = out != 0x8000
    assert np.array_equal(out[keep], out_z[keep])


@pytest.mark.parametrize("W", [2, 8, 16, 64])
def test_recursive_summation_error_bound(oracle_mod, W):
    """|a - exact| <= gamma_{W-1} * sum |x_r| with gamma_n = n u / (1 - n u), u = 2^-24
    (recursive summation bound, Higham, Accuracy and Stability of Numerical Algorithms)."""
    parts, _, _ = _rand_inputs(W, 4, 128, "fp32", 11, scale=3.0)
    # Mixed magnitudes to make rounding happen.
    parts = [p * np.float32(2.0 ** ((k % 7) - 3)) for k, p in enumerate(parts)]
    out = oracle_mod.ar_sum(parts, "fp32").astype(np.float64)
    stack = np.stack([p.astype(np.float64) for p in parts])
    exact = np.array([[math.fsum(stack[:, m, i]) for i in range(stack.shape[2])]
                      for m in range(stack.shape[1])])
    u = 2.0 ** -24
    g = (W - 1) * u / (1 - (W - 1) * u)
    bound = g * np.abs(stack).sum(axis=0)
    assert (np.abs(out - exact) <= bound * (1 + 1e-12)).all()
    assert (out != exact).any()  # the test data does exercise rounding


@pytest.mark.parametrize("dtype", DTYPES)
def test_brute_force_exact_rational_replay(oracle_mod, dtype):
    """Tiny shapes replayed with exact rationals: a = x_0, then a = RN_32(a + x_r) for each rank,
    then the residual, then RN_T -- rounding written from the IEEE definition in exact_arith,
    independent of the oracle's converters."""
    rng = np.random.default_rng(5)
    for trial in range(6):
        W = int(rng.integers(1, 5))
        M = int(rng.integers(1, 4))
        H = int(rng.integers(1, 17))
        scales = 2.0 ** rng.integers(-12, 12, size=W + 1)
        parts = [_store(rng.standard_normal((M, H)) * scales[k], dtype) for k in range(W)]
        res = _store(rng.standard_normal((M, H)) * scales[W], dtype)
        gam = np.ones(H, dtype=np.float32)
        out = oracle_mod.ar_sum(parts, dtype)
        ro, _ = oracle_mod.ar_residual_rmsnorm(parts, res, gam, 1e-6, dtype)
        bits = (lambda a: a.view(np.uint32)) if dtype == "fp32" else (lambda a: a)
        for m in range(M):
            for i in range(H):
                xs = [from_bits(int(bits(p)[m, i]), dtype) for p in parts]
                a = xs[0]
                for x in xs[1:]:
                    a = round_nearest_even(a + x, "fp32")
                assert int(bits(out)[m, i]) == to_bits(round_nearest_even(a, dtype), dtype) or \
                    (a == 0 and int(bits(out)[m, i]) & 0x7FFFFFFF == 0)
                a = round_nearest_even(a + from_bits(int(bits(res)[m, i]), dtype), "fp32")
                got = int(bits(ro)[m, i])
                assert got == to_bits(round_nearest_even(a, dtype), dtype) or \
                    (a == 0 and got & 0x7FFFFFFF == 0)


@pytest.mark.parametrize("dtype", DTYPES)
def test_residual_single_rank_is_textbook_add(oracle_mod, dtype):
    """W = 1: residual_out = RN_T(x_0 + residual), the plain add, computed here with torch."""
    parts, res, gam = _rand_inputs(1, 4, 96, dtype, 13)
    ro, _ = oracle_mod.ar_residual_rmsnorm(parts, res, gam, 1e-6, dtype)
    tx = torch.from_numpy(_values(parts[0], dtype)).float()
    tr = torch.from_numpy(_values(res, dtype)).float()
    want = synth.storage_numpy((tx + tr).to(TD[dtype]))
    assert np.array_equal(ro, want)


def test_residual_enters_after_partials(oracle_mod):
    """fp32: partials 2^24, 1 and residual 1 -> ((2^24 + 1) + 1) = 2^24 in the chain."""
    x0 = np.full((1, 4), 2.0 ** 24, dtype=np.float32)
    x1 = np.ones((1, 4), dtype=np.float32)
    ro, _ = oracle_mod.ar_residual_rmsnorm([x0, x1], x1.copy(), np.ones(4, np.float32), 0.0,
                                           "fp32")
    assert (ro == 2.0 ** 24).all()
    # Residual first in the chain would give 1 + 1 + 2^24 = 2^24 + 2: the oracle must not.
    ro2, _ = oracle_mod.ar_residual_rmsnorm([x1, x1.copy()], x0, np.ones(4, np.float32), 0.0,
                                            "fp32")
    assert (ro2 == 2.0 ** 24 + 2).all()


def test_row_range_only_touches_its_rows(oracle_mod):
    parts, res, gam = _rand_inputs(2, 6, 32, "bf16", 17)
    full = oracle_mod.ar_sum(parts, "bf16")
    part = np.full_like(full, 0xABCD)
    oracle_mod.ar_sum(parts, "bf16", rows=(2, 4), out=part)
    assert np.array_equal(part[2:4], full[2:4])
    assert (part[:2] == 0xABCD).all() and (part[4:] == 0xABCD).all()
