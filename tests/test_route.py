"""Routing policy (host only): the pages' decision rules as the library implements them.

* unsupported world sizes (12, 3, ...) go to the caller's fallback; norm rows the fused kernel
  does not take (odd widths, rows past its limit) go to the library's two-kernel path;
* below the token threshold (32 by default) every call stays one-shot;
* from the two-shot payload threshold on, two-shot; a per-rank payload cutoff sends larger
  calls to the fallback;
* the decision is monotone in M for a fixed policy (one-shot, then two-shot, then fallback).
"""
import pytest

import all_reduce_residual_amd as ar

ONE, TWO, FB, UNF = ar.ROUTE_ONE_SHOT, ar.ROUTE_TWO_SHOT, ar.ROUTE_FALLBACK, ar.ROUTE_UNFUSED
RMS, SUM, BF16 = ar.PATTERN_AR_RESIDUAL_RMSNORM, ar.PATTERN_ALLREDUCE, ar.DTYPE_BF16


def test_default_policy_values():
    p8 = ar.ar_policy_default(8)
    assert p8["min_tokens"] == 32 and p8["max_payload_bytes"] == 0
    # 5 us * 153 GB/s / (1 - 2/8) = 1.02 MB
    assert abs(p8["two_shot_min_bytes"] - 1_020_000) <= 1
    assert ar.ar_policy_default(2)["two_shot_min_bytes"] == 2 ** 63 - 1
    # Larger worlds cross over earlier.
    t = [ar.ar_policy_default(w)["two_shot_min_bytes"] for w in (4, 8, 16, 64)]
    assert t == sorted(t, reverse=True)


def test_world_size_twelve_falls_back():
    for pat in (SUM, RMS):
        assert ar.ar_route(pat, 12, 256, 7168, BF16) == FB
        assert ar.ar_route(pat, 3, 256, 7168, BF16) == FB
        assert ar.ar_route(pat, 8, 256, 7168, BF16) != FB


def test_norm_rows_the_fused_kernel_rejects_take_the_two_kernel_path():
    assert ar.ar_route(RMS, 8, 64, 7170, BF16) == UNF      # not whole 16-byte vectors
    assert ar.ar_route(RMS, 8, 1, 7170, BF16) == UNF       # at any token count
    assert ar.ar_route(RMS, 8, 4, 65544, BF16) == UNF      # wider than the fused limit
    assert ar.ar_route(RMS, 8, 4, 32772, ar.DTYPE_FP32) == UNF
    assert ar.ar_route(SUM, 8, 64, 7170, BF16) == ONE      # the sum kernel takes any H
    assert ar.ar_route(RMS, 12, 64, 7170, BF16) == FB      # world size still decides first
    pol = dict(min_tokens=32, two_shot_min_bytes=1 << 20, max_payload_bytes=1 << 20)
    assert ar.ar_route(RMS, 8, 1024, 7170, BF16, pol) == FB   # payload cutoff applies too


def test_token_threshold_and_payload():
    # Decode sizes: one-shot regardless of bytes.
    for M in (1, 8, 31):
        assert ar.ar_route(RMS, 8, M, 65536, BF16) == ONE
    # M >= 32 with a large payload: two-shot.
    assert ar.ar_route(RMS, 8, 2048, 7168, BF16) == TWO
    # M >= 32 but a small payload (32 x 256 x 2 = 16 KiB): one-shot.
    assert ar.ar_route(RMS, 8, 32, 256, BF16) == ONE
    # W = 2 never takes two-shot by default.
    assert ar.ar_route(RMS, 2, 4096, 8192, BF16) == ONE


def test_payload_cutoff_sends_to_fallback():
    pol = dict(min_tokens=32, two_shot_min_bytes=1 << 20, max_payload_bytes=80 << 20)
    assert ar.ar_route(SUM, 4, 5120, 8192, BF16, pol) == TWO      # 80 MiB: at the cutoff
    assert ar.ar_route(SUM, 4, 5121, 8192, BF16, pol) == FB       # one row more: above it


def test_monotone_in_tokens():
    pol = dict(min_tokens=32, two_shot_min_bytes=1 << 20, max_payload_bytes=64 << 20)
    order = {ONE: 0, TWO: 1, FB: 2}
    for W in ar.SUPPORTED_W:
        prev = 0
        for M in range(0, 6000, 37):
            r = order[ar.ar_route(RMS, W, M, 7168, BF16, pol)]
            assert r >= prev
            prev = r


def test_route_rejects_bad_arguments():
    with pytest.raises(ar.ArError):
        ar.ar_route(7, 8, 32, 256, BF16)
    with pytest.raises(ar.ArError):
        ar.ar_route(RMS, 8, 32, 256, BF16, dict(min_tokens=-1, two_shot_min_bytes=0,
                                                max_payload_bytes=0))


def test_routed_entry_validates_before_any_launch():
    """The routed entry point on fake pointers: every case here returns before a launch (the
    pointers are never dereferenced)."""
    import ctypes
    L = ar.lib()
    bf16 = ar.DTYPE_BF16
    pol = ar.Policy(**ar.ar_policy_default(8))
    route = ctypes.c_int(-7)
    ins = (ctypes.c_void_p * 12)(*[0x1000000 * (j + 1) for j in range(12)])
    out = 0x40000000
    # World size 12: the fallback route, AR_ERR_UNSUPPORTED, *route set.
    st = L.ar_allreduce_routed(ar.PATTERN_ALLREDUCE, ins, 12, 64, 7168, bf16, None, None, 1e-6,
                               out, None, 0, ctypes.byref(pol), ctypes.byref(route), None)
    assert st == ar.AR_ERR_UNSUPPORTED and route.value == ar.ROUTE_FALLBACK
    # A payload above the policy's cutoff: fallback as well.
    small = ar.Policy(min_tokens=32, two_shot_min_bytes=0, max_payload_bytes=1024)
    route.value = -7
    st = L.ar_allreduce_routed(ar.PATTERN_ALLREDUCE, ins, 8, 64, 7168, bf16, None, None, 1e-6,
                               out, None, 0, ctypes.byref(small), ctypes.byref(route), None)
    assert st == ar.AR_ERR_UNSUPPORTED and route.value == ar.ROUTE_FALLBACK
    # Bad rank, null route, null policy, bad pattern.
    for rank in (-1, 8):
        route.value = -7
        st = L.ar_allreduce_routed(ar.PATTERN_ALLREDUCE, ins, 8, 64, 7168, bf16, None, None,
                                   1e-6, out, None, rank, ctypes.byref(pol), ctypes.byref(route),
                                   None)
        assert st == ar.AR_ERR_INVALID_ARG and route.value == -7
    assert L.ar_allreduce_routed(ar.PATTERN_ALLREDUCE, ins, 8, 64, 7168, bf16, None, None, 1e-6,
                                 out, None, 0, ctypes.byref(pol), None, None) == \
        ar.AR_ERR_INVALID_ARG
    assert L.ar_allreduce_routed(ar.PATTERN_ALLREDUCE, ins, 8, 64, 7168, bf16, None, None, 1e-6,
                                 out, None, 0, None, ctypes.byref(route), None) == \
        ar.AR_ERR_INVALID_ARG
    assert L.ar_allreduce_routed(7, ins, 8, 64, 7168, bf16, None, None, 1e-6, out, None, 0,
                                 ctypes.byref(pol), ctypes.byref(route), None) == \
        ar.AR_ERR_INVALID_ARG
    # Two-shot share (2048 rows of 7168 bf16 at W = 8) with a null partial or a null norm output:
    # rejected before the row pointers are formed.
    ins[3] = None
    route.value = -7
    st = L.ar_allreduce_routed(ar.PATTERN_ALLREDUCE, ins, 8, 2048, 7168, bf16, None, None, 1e-6,
                               out, None, 2, ctypes.byref(pol), ctypes.byref(route), None)
    assert st == ar.AR_ERR_INVALID_ARG and route.value == ar.ROUTE_TWO_SHOT
    ins[3] = 0x4000000
    st = L.ar_allreduce_routed(ar.PATTERN_AR_RESIDUAL_RMSNORM, ins, 8, 2048, 7168, bf16,
                               0x50000000, 0x60000000, 1e-6, out, None, 2, ctypes.byref(pol),
                               ctypes.byref(route), None)
    assert st == ar.AR_ERR_INVALID_ARG and route.value == ar.ROUTE_TWO_SHOT
