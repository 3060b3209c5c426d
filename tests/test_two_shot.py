"""Two-shot share, host side: the row partition (library and oracle) and the all-gather's
argument validation.  The partition must tile [0, M) in rank order with slice sizes that differ
by at most one, and the library's partition must equal the oracle's floor(j * M / W) definition.
"""
import ctypes

import numpy as np
import pytest

import all_reduce_residual_amd as ar

BF16, FP32 = ar.DTYPE_BF16, ar.DTYPE_FP32


def test_oracle_partition_tiles_rows(oracle_mod):
    for W in (1, 2, 3, 4, 7, 8, 16, 64):
        for M in list(range(0, 70)) + [2048, 5120, 123457]:
            spans = [oracle_mod.row_partition(W, M, j) for j in range(W)]
            pos = 0
            for b, c in spans:
                assert b == pos and c >= 0
                pos += c
            assert pos == M
            sizes = [c for _, c in spans]
            assert max(sizes) - min(sizes) <= 1


def test_library_partition_matches_oracle(oracle_mod):
    for W in ar.SUPPORTED_W:
        for M in list(range(0, 130)) + [2048, 5120, 2 ** 40 + 3]:
            for j in range(W):
                assert ar.ar_row_partition(W, M, j) == oracle_mod.row_partition(W, M, j)


def test_partition_rejects_bad_arguments():
    for args in [(0, 4, 0), (8, 4, 8), (8, 4, -1), (8, -1, 0), (65, 4, 0)]:
        with pytest.raises(ar.ArError):
            ar.ar_row_partition(*args)


def test_oracle_two_shot_equals_one_shot(oracle_mod):
    """Rows are independent: per-slice results gathered in rank order equal the full result."""
    import synth
    W, M, H = 4, 11, 64
    parts, res, gam = synth.custom(W, M, H, "bf16", seed=3)
    hp = [synth.storage_numpy(p) for p in parts]
    hr = synth.storage_numpy(res)
    full_ro, full_no = oracle_mod.ar_residual_rmsnorm(hp, hr, gam.numpy(), 1e-6, "bf16")
    ro_slices, no_slices = [], []
    for j in range(W):
        b, c = oracle_mod.row_partition(W, M, j)
        ro, no = oracle_mod.ar_residual_rmsnorm([p[b:b + c].copy() for p in hp],
                                                hr[b:b + c].copy(), gam.numpy(), 1e-6, "bf16")
        ro_slices.append(ro)
        no_slices.append(no)
    assert np.array_equal(oracle_mod.all_gather(ro_slices), full_ro)
    assert np.array_equal(oracle_mod.all_gather(no_slices), full_no)


def _ptrs(vals):
    return (ctypes.c_void_p * len(vals))(*vals)


def test_all_gather_validation_before_device():
    L = ar.lib()
    # M=8, H=64 bf16 -> each of 4 slices is 2 rows = 256 bytes.
    sl = [0x100000 + 0x1000 * j for j in range(4)]
    out = 0x800000
    assert L.ar_all_gather(_ptrs(sl[:3] + [0] * 9), 12, 8, 64, BF16, out, None) == \
        ar.AR_ERR_UNSUPPORTED
    assert L.ar_all_gather(None, 4, 8, 64, BF16, out, None) == ar.AR_ERR_INVALID_ARG
    assert L.ar_all_gather(_ptrs(sl), 4, 8, 64, BF16, None, None) == ar.AR_ERR_INVALID_ARG
    assert L.ar_all_gather(_ptrs([sl[0], 0, sl[2], sl[3]]), 4, 8, 64, BF16, out, None) == \
        ar.AR_ERR_INVALID_ARG
    assert L.ar_all_gather(_ptrs([sl[0] + 4] + sl[1:]), 4, 8, 64, BF16, out, None) == \
        ar.AR_ERR_MISALIGNED
    assert L.ar_all_gather(_ptrs(sl), 4, 8, 64, BF16, out + 8, None) == ar.AR_ERR_MISALIGNED
    assert L.ar_all_gather(_ptrs(sl), 4, 8, 60, BF16, out, None) == ar.AR_ERR_UNSUPPORTED
    assert L.ar_all_gather(_ptrs(sl), 4, 8, 64, 7, out, None) == ar.AR_ERR_INVALID_ARG
    # A slice overlapping `out` somewhere other than its own place.
    assert L.ar_all_gather(_ptrs([out + 256] + sl[1:]), 4, 8, 64, BF16, out, None) == \
        ar.AR_ERR_ALIAS
    # Zero rows: nothing to do, no device access.
    assert L.ar_all_gather(None, 4, 0, 64, BF16, None, None) == ar.AR_OK
