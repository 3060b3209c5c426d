"""Helpers for the GPU tests: device copies, oracle runs and the comparison rules.

Comparison rules (the acceptance bar for the HIP path against the oracle):
  * out (kAllReduce) and residual_out: bit-identical, NaN matching NaN;
  * norm_out, 16-bit types: at most 1 unit in the last place apart (monotone integer order of
    the bit patterns, so +0 and -0 coincide and the largest finite value neighbours infinity);
  * norm_out, binary32: relative error at most 1e-5 (the rank sum itself stays bit-identical).
"""
from __future__ import annotations

import numpy as np
import torch

import synth

NORM_ULP_16BIT = 1
NORM_REL_FP32 = 1e-5


def dev(t: torch.Tensor) -> torch.Tensor:
    return t.to("cuda", non_blocking=False).contiguous()


def host_np(t: torch.Tensor) -> np.ndarray:
    return synth.storage_numpy(t)


def bits(a: np.ndarray) -> np.ndarray:
    return a.view(np.uint32) if a.dtype == np.float32 else a


def is_nan_bits(b: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "fp32":
        return ((b & 0x7F800000) == 0x7F800000) & ((b & 0x007FFFFF) != 0)
    if dtype == "bf16":
        return ((b & 0x7F80) == 0x7F80) & ((b & 0x007F) != 0)
    return ((b & 0x7C00) == 0x7C00) & ((b & 0x03FF) != 0)


def assert_bit_exact(got: np.ndarray, want: np.ndarray, dtype: str, what: str):
    g, w = bits(got), bits(want)
    nan_g, nan_w = is_nan_bits(g, dtype), is_nan_bits(w, dtype)
    ok = (g == w) | (nan_g & nan_w)
    if not ok.all():
        idx = np.argwhere(~ok)
        first = tuple(idx[0])
        raise AssertionError("%s: %d of %d elements differ; first at %s: got %#x want %#x" % (
            what, len(idx), ok.size, first, int(g[first]), int(w[first])))


def _ordered16(b: np.ndarray) -> np.ndarray:
    b = b.astype(np.int32)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def assert_norm_close(got: np.ndarray, want: np.ndarray, dtype: str, what: str = "norm_out"):
    if dtype == "fp32":
        nan_g, nan_w = np.isnan(got), np.isnan(want)
        assert (nan_g == nan_w).all(), "%s: NaN pattern differs" % what
        g = got[~nan_w].astype(np.float64)
        w = want[~nan_w].astype(np.float64)
        inf = np.isinf(w)
        assert (g[inf] == w[inf]).all(), "%s: infinities differ" % what
        err = np.abs(g[~inf] - w[~inf]) / np.maximum(np.abs(w[~inf]), 1e-30)
        worst = float(err.max()) if err.size else 0.0
        assert worst <= NORM_REL_FP32, "%s: max relative error %.3g > %g" % (
            what, worst, NORM_REL_FP32)
        return worst
    nan_g, nan_w = is_nan_bits(got, dtype), is_nan_bits(want, dtype)
    assert (nan_g == nan_w).all(), "%s: NaN pattern differs" % what
    d = np.abs(_ordered16(got[~nan_w]) - _ordered16(want[~nan_w]))
    worst = int(d.max()) if d.size else 0
    if worst > NORM_ULP_16BIT:
        i = int(np.argmax(d))
        raise AssertionError("%s: %d ulp apart at flat index %d (got %#x want %#x)" % (
            what, worst, i, int(got[~nan_w][i]), int(want[~nan_w][i])))
    return worst


def dtype_name(t: torch.dtype) -> str:
    return {torch.float32: "fp32", torch.float16: "fp16", torch.bfloat16: "bf16"}[t]
