"""Python access to the CPU oracle (``ar_oracle.cpp``) -- TEST INFRASTRUCTURE ONLY.

The oracle is the plain, slow definition of what the fused all-reduce-sum (+ residual + RMSNorm)
path computes.  Only the test suite, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this module.  The product package never imports it, and it imports nothing from
the product package.

Arrays are numpy arrays on the host.  16-bit storage types are carried as ``np.uint16`` bit
patterns (numpy has no bfloat16); binary32 as ``np.float32``.  Storage type codes:
``"fp32"``, ``"fp16"``, ``"bf16"``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ar_oracle.cpp")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

DTYPE_CODES = {"fp32": 0, "fp16": 1, "bf16": 2}

_lib = None
_lock = threading.Lock()


def build(force: bool = True) -> str:
    """Compile the oracle with g++ into ``oracle/liboracle.so`` and return its path.

    No -ffast-math and no FMA contraction: plain x86-64 SSE arithmetic with IEEE rounding,
    gradual underflow and no excess precision.
    """
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-o", tmp, _SRC]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        lib.oracle_round_f32_to_bf16.argtypes = [ctypes.c_float]
        lib.oracle_round_f32_to_bf16.restype = ctypes.c_uint16
        lib.oracle_round_f32_to_f16.argtypes = [ctypes.c_float]
        lib.oracle_round_f32_to_f16.restype = ctypes.c_uint16
        lib.oracle_widen_bf16.argtypes = [ctypes.c_uint16]
        lib.oracle_widen_bf16.restype = ctypes.c_float
        lib.oracle_widen_f16.argtypes = [ctypes.c_uint16]
        lib.oracle_widen_f16.restype = ctypes.c_float
        lib.oracle_round_f32_array.argtypes = [i32, vp, vp, i64]
        lib.oracle_round_f32_array.restype = i32
        lib.oracle_widen_array.argtypes = [i32, vp, vp, i64]
        lib.oracle_widen_array.restype = i32
        lib.oracle_ar_sum_rows.argtypes = [vp, i32, i64, i64, i32, vp, i64, i64]
        lib.oracle_ar_sum_rows.restype = i32
        lib.oracle_ar_residual_rmsnorm_rows.argtypes = [
            vp, i32, i64, i64, i32, vp, vp, ctypes.c_float, vp, vp, vp, vp, i64, i64]
        lib.oracle_ar_residual_rmsnorm_rows.restype = i32
        lib.oracle_rmsnorm_rows.argtypes = [vp, i64, i64, i32, vp, ctypes.c_float, vp, vp, vp,
                                            i64, i64]
        lib.oracle_rmsnorm_rows.restype = i32
        _lib = lib
        return lib


def _storage_np(dtype: str):
    return np.float32 if dtype == "fp32" else np.uint16


def _check_array(a: np.ndarray, dtype: str, shape) -> np.ndarray:
    if a.dtype != _storage_np(dtype):
        raise TypeError("expected %s storage for %s, got %s" % (_storage_np(dtype), dtype, a.dtype))
    if tuple(a.shape) != tuple(shape):
        raise ValueError("expected shape %s, got %s" % (shape, a.shape))
    if not a.flags["C_CONTIGUOUS"]:
        raise ValueError("arrays must be C-contiguous")
    return a


def _ptr_array(arrays):
    return (ctypes.c_void_p * len(arrays))(*[a.ctypes.data for a in arrays])


# ---- conversions --------------------------------------------------------------------------

def round_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    """binary32 -> bf16/fp16 bit patterns, round-to-nearest-even (the oracle's own converter)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty(x.shape, dtype=np.uint16)
    rc = _load().oracle_round_f32_array(DTYPE_CODES[dtype], x.ctypes.data, y.ctypes.data, x.size)
    if rc != 0:
        raise ValueError("bad dtype %r" % dtype)
    return y


def widen(b: np.ndarray, dtype: str) -> np.ndarray:
    """bf16/fp16 bit patterns -> binary32 values (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    y = np.empty(b.shape, dtype=np.float32)
    rc = _load().oracle_widen_array(DTYPE_CODES[dtype], b.ctypes.data, y.ctypes.data, b.size)
    if rc != 0:
        raise ValueError("bad dtype %r" % dtype)
    return y


def to_f32(a: np.ndarray, dtype: str) -> np.ndarray:
    """Storage array (any type) -> binary32 values."""
    return a.astype(np.float32) if dtype == "fp32" else widen(a, dtype)


# ---- the two patterns ---------------------------------------------------------------------

def ar_sum(inputs, dtype: str, rows=None, out=None) -> np.ndarray:
    """kAllReduce: out = rank-ordered binary32 sum of the W partials, rounded once to dtype.

    ``inputs`` is a list of W arrays [M, H].  ``rows`` = (row0, row1) restricts the work to
    those rows (the other rows of ``out`` are left as they were).
    """
    W = len(inputs)
    if W < 1:
        raise ValueError("need at least one partial")
    M, H = inputs[0].shape
    for a in inputs:
        _check_array(a, dtype, (M, H))
    if out is None:
        out = np.zeros((M, H), dtype=_storage_np(dtype))
    _check_array(out, dtype, (M, H))
    r0, r1 = (0, M) if rows is None else rows
    rc = _load().oracle_ar_sum_rows(_ptr_array(inputs), W, M, H, DTYPE_CODES[dtype],
                                    out.ctypes.data, r0, r1)
    if rc != 0:
        raise ValueError("oracle_ar_sum rejected its arguments")
    return out


def ar_residual_rmsnorm(inputs, residual, gamma, eps: float, dtype: str, rows=None,
                        residual_out=None, norm_out=None, debug: bool = False):
    """kARResidualRMSNorm.

    Returns ``(residual_out, norm_out)``, or ``(residual_out, norm_out, y, rstd)`` with
    ``debug=True`` (``y`` [M, H] float64 = unrounded normalised and scaled values, ``rstd`` [M]
    float64).  ``rows`` = (row0, row1) restricts the work to those rows.
    """
    W = len(inputs)
    if W < 1:
        raise ValueError("need at least one partial")
    M, H = inputs[0].shape
    for a in inputs:
        _check_array(a, dtype, (M, H))
    _check_array(residual, dtype, (M, H))
    gamma = np.ascontiguousarray(gamma, dtype=np.float32)
    if gamma.shape != (H,):
        raise ValueError("gamma must be [H] float32")
    sdt = _storage_np(dtype)
    if residual_out is None:
        residual_out = np.zeros((M, H), dtype=sdt)
    if norm_out is None:
        norm_out = np.zeros((M, H), dtype=sdt)
    _check_array(residual_out, dtype, (M, H))
    _check_array(norm_out, dtype, (M, H))
    y = np.full((M, H), np.nan) if debug else None
    rstd = np.full((M,), np.nan) if debug else None
    r0, r1 = (0, M) if rows is None else rows
    rc = _load().oracle_ar_residual_rmsnorm_rows(
        _ptr_array(inputs), W, M, H, DTYPE_CODES[dtype], residual.ctypes.data,
        gamma.ctypes.data, float(eps), residual_out.ctypes.data, norm_out.ctypes.data,
        y.ctypes.data if debug else None, rstd.ctypes.data if debug else None, r0, r1)
    if rc != 0:
        raise ValueError("oracle_ar_residual_rmsnorm rejected its arguments")
    if debug:
        return residual_out, norm_out, y, rstd
    return residual_out, norm_out


def rmsnorm(x, gamma, eps: float, dtype: str, rows=None, out=None, debug: bool = False):
    """RMSNorm of a stored [M, H] tensor (the normalisation step of kARResidualRMSNorm alone).

    Returns ``out``, or ``(out, y, rstd)`` with ``debug=True``.
    """
    M, H = x.shape
    _check_array(x, dtype, (M, H))
    gamma = np.ascontiguousarray(gamma, dtype=np.float32)
    if gamma.shape != (H,):
        raise ValueError("gamma must be [H] float32")
    if out is None:
        out = np.zeros((M, H), dtype=_storage_np(dtype))
    _check_array(out, dtype, (M, H))
    y = np.full((M, H), np.nan) if debug else None
    rstd = np.full((M,), np.nan) if debug else None
    r0, r1 = (0, M) if rows is None else rows
    rc = _load().oracle_rmsnorm_rows(
        x.ctypes.data, M, H, DTYPE_CODES[dtype], gamma.ctypes.data, float(eps), out.ctypes.data,
        y.ctypes.data if debug else None, rstd.ctypes.data if debug else None, r0, r1)
    if rc != 0:
        raise ValueError("oracle_rmsnorm rejected its arguments")
    if debug:
        return out, y, rstd
    return out


# ---- two-shot share --------------------------------------------------------------------------

def row_partition(W: int, M: int, rank: int):
    """(row_begin, row_count) of `rank` in the W-way split of M rows: row_begin(j) = floor(j*M/W)."""
    if not (1 <= W and 0 <= rank < W and M >= 0):
        raise ValueError("bad partition arguments")
    b = (rank * M) // W
    e = ((rank + 1) * M) // W
    return b, e - b


def all_gather(slices) -> np.ndarray:
    """The gathered tensor: the W row slices stacked in rank order."""
    return np.concatenate(list(slices), axis=0)
