"""Pins of the oracle's own storage-type conversions (host only).

The oracle rounds binary32 to bfloat16 / binary16 with its own code.  These tests hold it to
library routines that implement the same IEEE round-to-nearest-even: torch's bfloat16 cast and
numpy's float16 cast, over
  * every 16-bit pattern for the widening direction (exhaustive),
  * every (sign, exponent, top significand bits) combination crossed with all low-bit patterns
    that decide a rounding (exact tie, one below, one above, all ones, zero) at every rounding
    position the format can have (normal and subnormal targets),
  * a random sample of binary32 patterns,
  * every binary32 pattern (exhaustive, 2^32 inputs in parallel chunks, ~30 s),
and to hand-derived IEEE cases (ties to even, overflow, gradual underflow).
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

from exact_arith import f32_value, round_nearest_even, to_bits

RNG = np.random.default_rng(20261202)


def _torch_bf16_bits(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _numpy_f16_bits(x: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore", invalid="ignore"):
        return x.astype(np.float16).view(np.uint16)


def _assert_same_rounding(got: np.ndarray, want: np.ndarray, x: np.ndarray, fmt: str):
    nan_x = np.isnan(x)
    ok = (got == want) | nan_x
    if not ok.all():
        bad = np.flatnonzero(~ok)[:10]
        msg = ", ".join("%08x -> %04x (want %04x)" % (x.view(np.uint32)[i], got[i], want[i])
                        for i in bad)
        pytest.fail("%s rounding mismatches: %s" % (fmt, msg))
    # NaN must stay NaN (payload is not compared).
    exp_mask = 0x7F80 if fmt == "bf16" else 0x7C00
    man_mask = 0x007F if fmt == "bf16" else 0x03FF
    g = got[nan_x]
    assert ((g & exp_mask) == exp_mask).all() and ((g & man_mask) != 0).all()


def _critical_patterns():
    """binary32 patterns that exercise every rounding decision for both narrow formats."""
    out = []
    signs = np.array([0, 1], dtype=np.uint32) << 31
    exps = np.arange(256, dtype=np.uint32) << 23
    se = (signs[:, None] | exps[None, :]).reshape(-1)                 # 512 sign/exponent pairs
    # Top 10 significand bits x low-13-bit rounding patterns (binary16 normal targets, and
    # bfloat16 at every top-7 value since its rounding point is bit 16).
    top10 = np.arange(1024, dtype=np.uint32) << 13
    low13 = np.array([0, 1, 0x0FFF, 0x1000, 0x1001, 0x1FFF], dtype=np.uint32)
    m = (top10[:, None] | low13[None, :]).reshape(-1)
    out.append((se[:, None] | m[None, :]).reshape(-1))
    # bfloat16 rounding point (bit 16) with every top-7 value and random bits above.
    top7 = np.arange(128, dtype=np.uint32) << 16
    low16 = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint32)
    m = (top7[:, None] | low16[None, :]).reshape(-1)
    out.append((se[:, None] | m[None, :]).reshape(-1))
    # Every other rounding position p (binary16 subnormal targets drop more bits): bits below p
    # in {0, 1, half-1, half, half+1, all ones}, random bits above p.
    for p in range(1, 24):
        half = np.uint32(1 << (p - 1))
        below = np.array([0, 1, half - 1, half, half + 1, (1 << p) - 1], dtype=np.uint32)
        hi = RNG.integers(0, 1 << 23, size=32, dtype=np.uint32) & ~np.uint32((1 << p) - 1)
        m = (hi[:, None] | below[None, :]).reshape(-1) & np.uint32(0x7FFFFF)
        out.append((se[:, None] | m[None, :]).reshape(-1))
    return np.unique(np.concatenate(out)).view(np.float32)


CRITICAL = _critical_patterns()
SAMPLE = RNG.integers(0, 1 << 32, size=1 << 22, dtype=np.uint64).astype(np.uint32).view(np.float32)


@pytest.mark.parametrize("xs", [CRITICAL, SAMPLE], ids=["critical", "random"])
def test_round_bf16_matches_torch(oracle_mod, xs):
    _assert_same_rounding(oracle_mod.round_f32(xs, "bf16"), _torch_bf16_bits(xs), xs, "bf16")


@pytest.mark.parametrize("xs", [CRITICAL, SAMPLE], ids=["critical", "random"])
def test_round_f16_matches_numpy(oracle_mod, xs):
    _assert_same_rounding(oracle_mod.round_f32(xs, "fp16"), _numpy_f16_bits(xs), xs, "fp16")


def test_round_exhaustive_every_binary32(oracle_mod):
    """All 2^32 binary32 patterns through both of the oracle's rounding converters, against
    torch's bfloat16 and float16 casts (IEEE round to nearest even, subnormals kept, overflow
    to infinity); NaN inputs must give NaN."""
    chunk = 1 << 24

    def check(i):
        x = np.arange(i * chunk, (i + 1) * chunk, dtype=np.uint64).astype(np.uint32)
        x = x.view(np.float32)
        nan = np.isnan(x)
        bad = 0
        for fmt, tdt in (("bf16", torch.bfloat16), ("fp16", torch.float16)):
            got = oracle_mod.round_f32(x, fmt)
            want = torch.from_numpy(x).to(tdt).view(torch.int16).numpy().view(np.uint16)
            bad += int((~((got == want) | nan)).sum())
            exp_mask, man_mask = (0x7F80, 0x007F) if fmt == "bf16" else (0x7C00, 0x03FF)
            g = got[nan]
            bad += int((~(((g & exp_mask) == exp_mask) & ((g & man_mask) != 0))).sum())
        return bad

    with ThreadPoolExecutor(max_workers=8) as pool:
        mismatches = sum(pool.map(check, range((1 << 32) // chunk)))
    assert mismatches == 0


def test_critical_set_covers_every_exponent():
    e = (CRITICAL.view(np.uint32) >> 23) & 0xFF
    assert len(np.unique(e)) == 256
    assert len(CRITICAL) > 1_000_000


def test_widen_bf16_exhaustive(oracle_mod):
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle_mod.widen(b, "bf16")
    want = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).float().numpy()
    nan = np.isnan(want)
    assert (np.isnan(got) == nan).all()
    assert (got.view(np.uint32)[~nan] == want.view(np.uint32)[~nan]).all()


def test_widen_f16_exhaustive(oracle_mod):
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle_mod.widen(b, "fp16")
    want = b.view(np.float16).astype(np.float32)
    nan = np.isnan(want)
    assert (np.isnan(got) == nan).all()
    assert (got.view(np.uint32)[~nan] == want.view(np.uint32)[~nan]).all()


# Hand-derived IEEE cases: (binary32 input, expected 16-bit pattern).
HAND_BF16 = [
    (1.0 + 2.0 ** -8, 0x3F80),               # exact tie between 1 and 1+2^-7: even -> 1
    (1.0 + 3 * 2.0 ** -8, 0x3F82),           # tie between 1+2^-7 (odd) and 1+2^-6: -> 1+2^-6
    (1.0 + 2.0 ** -8 + 2.0 ** -20, 0x3F81),  # just above the tie -> up
    (-0.0, 0x8000),
    (3.3895313892515355e38, 0x7F7F),         # largest bfloat16 finite value
    (3.3961775292304957e38, 0x7F80),         # its midpoint to 2^128 rounds to even: infinity
    (2.0 ** -133, 0x0001),                   # smallest bfloat16 subnormal
    (2.0 ** -134, 0x0000),                   # half of it: tie to even zero
    (3 * 2.0 ** -134, 0x0002),               # 1.5 quanta: tie to even 2
]
HAND_F16 = [
    (65504.0, 0x7BFF),                       # largest binary16 finite
    (65519.99609375, 0x7BFF),                # just below the midpoint
    (65520.0, 0x7C00),                       # midpoint to 2^16 rounds to even: infinity
    (1.0 + 2.0 ** -11, 0x3C00),              # tie -> even
    (1.0 + 3 * 2.0 ** -11, 0x3C02),
    (2.0 ** -24, 0x0001),                    # smallest subnormal
    (2.0 ** -25, 0x0000),                    # tie to even zero
    (3 * 2.0 ** -25, 0x0002),                # tie to even 2
    (2.0 ** -14 - 2.0 ** -24, 0x03FF),       # largest subnormal
    (-(2.0 ** -14), 0x8400),                 # smallest normal, negative
]


@pytest.mark.parametrize("x,bits", HAND_BF16)
def test_round_bf16_hand_cases(oracle_mod, x, bits):
    got = int(oracle_mod.round_f32(np.array([x], dtype=np.float32), "bf16")[0])
    assert got == bits
    if x == 0.0:
        return  # Fraction has no signed zero
    # And the exact-rational definition agrees.
    v = round_nearest_even(f32_value(int(np.array([x], np.float32).view(np.uint32)[0])), "bf16")
    assert to_bits(v, "bf16") == bits


@pytest.mark.parametrize("x,bits", HAND_F16)
def test_round_f16_hand_cases(oracle_mod, x, bits):
    got = int(oracle_mod.round_f32(np.array([x], dtype=np.float32), "fp16")[0])
    assert got == bits
    if x == 0.0:
        return
    v = round_nearest_even(f32_value(int(np.array([x], np.float32).view(np.uint32)[0])), "fp16")
    assert to_bits(v, "fp16") == bits
