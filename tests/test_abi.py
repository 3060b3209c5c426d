"""Host-only checks of the C ABI library: it loads, exports every function include/ar_fused.h
declares, and its host logic (shape checks, status strings, the launch-shape heuristic and
argument validation that rejects before any device access) behaves as documented.  No call here
reaches the device: every entry-point call is one the library must reject during validation.
"""
import ctypes
import itertools

import pytest

import all_reduce_residual_amd as ar

BF16, FP16, FP32 = ar.DTYPE_BF16, ar.DTYPE_FP16, ar.DTYPE_FP32
RMS, SUM = ar.PATTERN_AR_RESIDUAL_RMSNORM, ar.PATTERN_ALLREDUCE


@pytest.fixture(scope="module")
def L():
    return ar.lib()


def test_exports_every_declared_function(L):
    names = ar.header_functions()
    assert set(names) == {"ar_sum", "ar_residual_rmsnorm", "ar_supports", "ar_launch_config",
                          "ar_residual_rmsnorm_noalloc", "ar_sum_with_config",
                          "ar_residual_rmsnorm_with_config",
                          "ar_status_string", "ar_device_cu_count", "ar_row_partition",
                          "ar_all_gather", "ar_lamport_arm", "ar_lamport_push",
                          "ar_lamport_sum", "ar_lamport_residual_rmsnorm",
                          "ar_policy_default", "ar_route", "ar_allreduce_routed", "ar_rmsnorm",
                          "ar_residual_rmsnorm_unfused", "ar_split_workspace_bytes",
                          "ar_workspace_clear", "ar_split_config", "ar_residual_rmsnorm_ws",
                          "ar_residual_rmsnorm_split_with_config"}
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    seen = set()
    for code in range(7):
        s = ar.status_string(code)
        assert s and s != "unknown status"
        seen.add(s)
    assert len(seen) == 7
    assert ar.status_string(99) == "unknown status"


def test_supports_world_sizes():
    for W in range(0, 70):
        st = ar.ar_supports(RMS, W, 4, 256, BF16)
        if W < 1:
            assert st == ar.AR_ERR_INVALID_ARG
        elif W in ar.SUPPORTED_W:
            assert st == ar.AR_OK, W
        else:
            assert st == ar.AR_ERR_UNSUPPORTED, W
    assert ar.ar_supports(SUM, 12, 4, 256, BF16) == ar.AR_ERR_UNSUPPORTED


def test_supports_shapes():
    assert ar.ar_supports(RMS, 8, 0, 7168, BF16) == ar.AR_OK
    assert ar.ar_supports(RMS, 8, -1, 7168, BF16) == ar.AR_ERR_INVALID_ARG
    assert ar.ar_supports(RMS, 8, 4, 0, BF16) == ar.AR_ERR_INVALID_ARG
    assert ar.ar_supports(RMS, 8, 4, 7168, 3) == ar.AR_ERR_INVALID_ARG
    assert ar.ar_supports(7, 8, 4, 7168, BF16) == ar.AR_ERR_INVALID_ARG
    assert ar.ar_supports(RMS, 8, 4, 7170, BF16) == ar.AR_ERR_UNSUPPORTED   # not a multiple of 8
    assert ar.ar_supports(SUM, 8, 4, 7170, BF16) == ar.AR_OK                # any size for sum
    assert ar.ar_supports(RMS, 8, 4, 1020, FP32) == ar.AR_OK                # multiple of 4
    assert ar.ar_supports(RMS, 8, 4, 65536, BF16) == ar.AR_OK
    assert ar.ar_supports(RMS, 8, 4, 65544, BF16) == ar.AR_ERR_UNSUPPORTED
    assert ar.ar_supports(RMS, 8, 4, 32768, FP32) == ar.AR_OK
    assert ar.ar_supports(RMS, 8, 4, 32772, FP32) == ar.AR_ERR_UNSUPPORTED
    assert ar.ar_supports(SUM, 8, 1 << 40, 1 << 30, BF16) == ar.AR_ERR_UNSUPPORTED
    # Huge M alone must not overflow the size check.
    assert ar.ar_supports(SUM, 8, (1 << 62) + 5, 1, FP32) == ar.AR_ERR_UNSUPPORTED
    assert ar.ar_supports(SUM, 8, 2 ** 63 - 1, 1, FP32) == ar.AR_ERR_UNSUPPORTED
    assert ar.ar_supports(SUM, 8, 1 << 59, 1, BF16) == ar.AR_OK           # 2^60 bytes exactly


SHAPES = list(itertools.product(
    [1, 2, 4, 8, 16, 32, 64], [1, 3, 4, 8, 31, 32, 33, 64, 128, 255, 256, 257, 512, 2048, 5120,
                               65536],
    [8, 64, 256, 520, 1016, 4096, 7168, 8192, 16384, 65536], [BF16, FP16, FP32]))


def _vec(dtype):
    return 4 if dtype == FP32 else 8


@pytest.mark.parametrize("cu", [256, 80, 304])
def test_launch_config_invariants(cu):
    for W, M, H, dt in SHAPES:
        for pat in (SUM, RMS):
            if ar.ar_supports(pat, W, M, H, dt) != ar.AR_OK:
                continue
            c = ar.ar_launch_config(pat, W, M, H, dt, cu_count=cu)
            assert c == ar.ar_launch_config(pat, W, M, H, dt, cu_count=cu)   # deterministic
            t = c["threads_per_block"]
            assert 64 <= t <= 1024 and t % 64 == 0, c
            assert c["nt_store"] in (0, 1)
            assert c["grid"] >= 1
            n = c["ranks_per_batch"]
            assert n in (0, 1, 2, 4)
            if n:
                # Only where it is built, one row per block, non-temporal stores: one rank per
                # batch at one to three rows per CU, two or four from there on.
                vpt = c["vecs_per_thread"]
                assert pat == RMS and c["nt_store"] == 1 and c["rows_per_block"] == 1, c
                assert _rank_batch_built(W, vpt, n), c
                assert (cu < M <= 3 * cu) if n == 1 else M > 3 * cu, c
            if pat == SUM:
                assert c["flat"] == 1 and c["vecs_per_thread"] in (1, 2, 4)
                nvec = M * H // _vec(dt)
                assert c["grid"] * t * c["vecs_per_thread"] >= nvec or c["grid"] == 2 ** 31 - 1
            else:
                L_, vpt, R = c["lanes_per_row"], c["vecs_per_thread"], c["rows_per_block"]
                assert c["flat"] == 0 and vpt in (1, 2, 4, 8)
                assert (L_ <= 64 and L_ & (L_ - 1) == 0) or L_ % 64 == 0
                assert t % L_ == 0 and R == t // L_
                assert L_ * vpt >= H // _vec(dt), c                     # row covered
                assert c["grid"] * R >= M                              # rows covered
                # No thread is idle for a whole row when the row fits the block (except the rows
                # kept at 8 vectors per thread: a single tensor once M >= 8 x CUs, two 16-bit
                # partials once M >= 4 x CUs).
                kept = (W == 1 and M >= 8 * cu) or (W == 2 and dt != FP32 and M // cu >= 4)
                assert L_ * vpt - H // _vec(dt) < L_ or L_ <= 64 or kept, c


def test_launch_config_headline_shapes():
    """The wide-hidden decode/prefill sweep (W=8, H=7168 bf16) keeps every CU busy as M grows."""
    for M in (1, 8, 32, 64, 128, 512, 2048):
        c = ar.ar_launch_config(RMS, 8, M, 7168, BF16, cu_count=256)
        assert c["grid"] == M and c["rows_per_block"] == 1
        assert c["lanes_per_row"] * c["vecs_per_thread"] >= 896


def _rank_batch_built(W, vpt, n):
    """The fixed rank batches the library is built with."""
    return ((n == 1 and ((vpt == 2 and 4 <= W <= 16) or (vpt == 4 and W in (2, 4)))) or
            (n == 2 and ((vpt == 2 and W >= 4) or (vpt == 1 and W >= 32))) or
            (n == 4 and vpt == 2 and W == 8))


def test_launch_config_rank_batch_bands():
    """Whole rows load one rank per batch while every row is resident with one to three rows per
    CU, then two ranks (four at W = 8 with 16-bit rows); never below one row per CU."""
    def rpb(W, M, H, dt, cu=256):
        return ar.ar_launch_config(RMS, W, M, H, dt, cu_count=cu)["ranks_per_batch"]
    for M, want in ((1, 0), (128, 0), (256, 0), (257, 1), (512, 1), (768, 1), (769, 4),
                    (1024, 4), (2048, 4), (8192, 4)):
        assert rpb(8, M, 7168, BF16) == want, M
    assert rpb(8, 2048, 8192, FP16) == 4
    assert rpb(16, 512, 8192, FP16) == 1 and rpb(16, 2048, 8192, FP16) == 2
    assert rpb(4, 512, 7168, BF16) == 1 and rpb(4, 2048, 7168, BF16) == 2
    assert rpb(8, 2048, 4096, FP32) == 2          # binary32 rows at W = 8: two ranks
    assert rpb(2, 512, 7168, BF16) == 1           # W = 2: 4 vectors
    assert rpb(2, 512, 4096, BF16) == 0           # W = 2 with 2 vectors: staged chains already
    assert rpb(2, 2048, 7168, BF16) == 0          # W = 2 keeps 8 vectors there
    assert rpb(32, 512, 7168, BF16) == 0 and rpb(1, 512, 7168, BF16) == 0
    assert rpb(32, 1024, 7168, BF16) == 2         # two vectors per thread
    assert rpb(32, 2048, 7168, BF16) == 2 and rpb(64, 4096, 7168, BF16) == 2   # one vector
    assert rpb(8, 2048, 4096, BF16) == 0          # one vector at W = 8: default batches
    assert rpb(64, 1024, 2048, FP32) == 0 and rpb(32, 2048, 2048, FP32) == 2   # binary32, 1 vector
    assert rpb(8, 160, 7168, BF16, cu=80) == 1 and rpb(8, 80, 7168, BF16, cu=80) == 0
    assert rpb(8, 241, 7168, BF16, cu=80) == 4
    for M in (1, 512, 2048):                      # never for the sum
        assert ar.ar_launch_config(SUM, 8, M, 7168, BF16, cu_count=256)["ranks_per_batch"] == 0


def test_launch_config_sum_resident_round():
    """Mid-size sums that 3/4 to 2 blocks of 256 threads per CU cover run as one resident round
    (one vector per thread for W <= 8, four for W >= 8); other sizes keep single-wave blocks."""
    def shape(W, M, H=7168):
        c = ar.ar_launch_config(SUM, W, M, H, BF16, cu_count=256)
        return c["threads_per_block"], c["vecs_per_thread"], c["grid"]
    assert shape(8, 64) == (256, 1, 224)
    assert shape(8, 128) == (256, 1, 448)
    assert shape(2, 128) == (256, 1, 448)
    assert shape(8, 512) == (256, 4, 448)
    assert shape(64, 512) == (256, 4, 448)
    assert shape(16, 512, 8192) == (256, 4, 512)
    assert shape(2, 512) == (64, 1, 7168)          # W <= 4: four vectors per thread lose
    assert shape(16, 128) == (64, 1, 1792)         # W >= 16: one vector per thread is mixed
    assert shape(8, 2048) == (64, 1, 28672)        # beyond one round
    assert shape(8, 8) == (64, 2, 56)              # too few blocks for the round
    assert shape(8, 256) == (64, 1, 3584)          # 8-16 single-wave blocks per CU: one vector
    assert shape(4, 160) == (64, 1, 2240)
    assert shape(8, 16) == (64, 2, 112)            # under 8 blocks per CU: two vectors
    # 16 or more ranks: the 4-vector blocks up to 8 blocks per CU.
    assert shape(32, 2048) == (256, 4, 1792)
    assert shape(16, 1024, 8192) == (256, 4, 1024)
    assert shape(64, 3072) == (64, 1, 43008)        # beyond 8 blocks per CU
    assert shape(8, 1024) == (64, 1, 14336)         # W = 8: up to 2 blocks per CU only
    # On a GPU with fewer CUs the bands move with the CU count.
    c = ar.ar_launch_config(SUM, 8, 128, 7168, BF16, cu_count=80)
    assert (c["threads_per_block"], c["vecs_per_thread"]) == (64, 1)
    c = ar.ar_launch_config(SUM, 8, 40, 7168, BF16, cu_count=80)
    assert (c["threads_per_block"], c["vecs_per_thread"], c["grid"]) == (256, 1, 140)


def test_launch_config_many_ranks_many_rows():
    """W >= 32 with 16-bit rows and at least 8 rows per CU: one vector per thread over the
    whole row; otherwise the two-vector rows of up to 512 lanes."""
    def shape(W, M, H=7168, dt=BF16, cu=256):
        c = ar.ar_launch_config(RMS, W, M, H, dt, cu_count=cu)
        return c["threads_per_block"], c["vecs_per_thread"]
    assert shape(32, 2048) == (896, 1)
    assert shape(64, 2048) == (896, 1)
    assert shape(32, 2048, 8192, FP16) == (1024, 1)
    assert shape(64, 4096, 16384) == (1024, 2)            # wider rows: the fewest vectors
    assert shape(32, 2047) == (448, 2)                    # under 8 rows per CU
    assert shape(16, 2048) == (448, 2)
    assert shape(32, 2048, 4096, FP32) == (512, 2)
    assert shape(32, 640, cu=80) == (896, 1)              # the bound moves with the CU count



def test_launch_config_binary32_rows_by_row_count():
    """Binary32 rows of 1025-2048 vectors: two vectors per thread over up to 1024 lanes while a
    quarter of the CUs or fewer hold a row, or from 8 rows per CU; four over up to 512 between,
    and narrower rows keep their shapes."""
    def shape(W, M, H=7168, cu=256):
        c = ar.ar_launch_config(RMS, W, M, H, FP32, cu_count=cu)
        return c["threads_per_block"], c["vecs_per_thread"]
    assert shape(8, 1) == (896, 2)
    assert shape(32, 64) == (896, 2)
    assert shape(8, 65) == (448, 4)                       # over a quarter of the CUs
    assert shape(8, 1024) == (448, 4)
    assert shape(8, 2047) == (448, 4)
    assert shape(8, 2048) == (896, 2)
    assert shape(2, 2048, 8192) == (1024, 2)              # W = 2's narrow rows give way too
    assert shape(8, 32, 5120) == (640, 2)
    assert shape(8, 1, 4096) == (512, 2)                  # 1024 vectors: unchanged
    assert shape(8, 1, 16384) == (512, 8)                 # 4096 vectors: unchanged
    assert shape(8, 20, cu=80) == (896, 2)                # the bounds move with the CU count
    assert shape(8, 21, cu=80) == (448, 4)
    c = ar.ar_launch_config(RMS, 8, 1, 7168, BF16, cu_count=256)
    assert (c["threads_per_block"], c["vecs_per_thread"]) == (448, 2)   # 16-bit: unchanged


def test_launch_config_many_ranks_widest_rows():
    """Eight or more partials on rows of over 2048 vectors: four vectors per thread while the row
    fits 768 lanes (1024 for W = 16); fewer partials and wider rows keep eight."""
    def shape(W, M, H, dt=BF16):
        c = ar.ar_launch_config(RMS, W, M, H, dt, cu_count=256)
        return c["threads_per_block"], c["vecs_per_thread"]
    assert shape(16, 1, 20480) == (640, 4)
    assert shape(16, 1024, 32768, FP16) == (1024, 4)
    assert shape(32, 1, 24576) == (768, 4)
    assert shape(64, 256, 20480) == (640, 4)
    assert shape(8, 64, 20480) == (640, 4)
    assert shape(32, 1, 32768) == (512, 8)                # over 768 lanes: eight
    assert shape(16, 1, 65536) == (1024, 8)               # over 1024 lanes at four
    assert shape(4, 1, 20480) == (320, 8)                 # fewer partials: unchanged
    assert shape(16, 1, 16384) == (512, 4)                # 2048 vectors: four already
    assert shape(16, 64, 12288, FP32) == (768, 4)         # binary32 at few rows
    assert shape(16, 65, 12288, FP32) == (384, 8)         # binary32 beyond: eight

def test_launch_config_two_partials_by_rows_per_cu():
    """W = 2: rows shrink with the rows per CU and keep 8 vectors per thread from 4 rows per CU
    (16-bit), then return to the W >= 4 shape from 12 rows per CU (16-bit); binary32 and a
    single tensor keep the narrow rows."""
    def shape(W, M, H=7168, dt=BF16, cu=256):
        c = ar.ar_launch_config(RMS, W, M, H, dt, cu_count=cu)
        return c["threads_per_block"], c["vecs_per_thread"]
    assert shape(2, 512) == (256, 4)                      # 2 rows per CU: halved, no idle slot
    assert shape(2, 1024) == (128, 8)                     # 4: 8 vectors kept (896 of 1024 slots)
    assert shape(2, 2048) == (128, 8)
    assert shape(2, 2048, 4096) == (64, 8)
    assert shape(2, 3072) == (448, 2)                     # 12: the W >= 4 shape
    assert shape(2, 8192, 4096) == (512, 1)
    assert shape(2, 4096, 8192, FP16) == (512, 2)
    assert shape(2, 4096, 3584, FP32) == (256, 4)         # binary32: narrow rows, halved
    assert shape(1, 4096) == (128, 8)                     # single tensor: unchanged


def test_launch_config_rejects():
    with pytest.raises(ar.ArError) as e:
        ar.ar_launch_config(RMS, 12, 4, 256, BF16, cu_count=256)
    assert e.value.status == ar.AR_ERR_UNSUPPORTED


def _ptrs(vals):
    return (ctypes.c_void_p * len(vals))(*vals)


def test_validation_rejects_before_device_access(L):
    """Every call below is invalid and must be rejected by host validation (fake pointers are
    never dereferenced)."""
    p = [0x10000 * (i + 1) for i in range(16)]   # 16-byte aligned, never touched
    out = 0x900000
    # World size 12.
    assert L.ar_sum(_ptrs(p[:12]), 12, 4, 256, BF16, out, None) == ar.AR_ERR_UNSUPPORTED
    assert L.ar_residual_rmsnorm(_ptrs(p[:12]), 12, 4, 256, BF16, 0xA00000, 0xB00000, 1e-6,
                                 0xC00000, 0xD00000, None) == ar.AR_ERR_UNSUPPORTED
    # Null input array / null partial / null output.
    assert L.ar_sum(None, 2, 4, 256, BF16, out, None) == ar.AR_ERR_INVALID_ARG
    assert L.ar_sum(_ptrs([p[0], 0]), 2, 4, 256, BF16, out, None) == ar.AR_ERR_INVALID_ARG
    assert L.ar_sum(_ptrs(p[:2]), 2, 4, 256, BF16, None, None) == ar.AR_ERR_INVALID_ARG
    # Misaligned.
    assert L.ar_sum(_ptrs([p[0] + 2, p[1]]), 2, 4, 256, BF16, out, None) == ar.AR_ERR_MISALIGNED
    assert L.ar_sum(_ptrs(p[:2]), 2, 4, 256, BF16, out + 8, None) == ar.AR_ERR_MISALIGNED
    # Partial overlap of out with an input (4*256*2 = 2048 bytes each).
    assert L.ar_sum(_ptrs(p[:2]), 2, 4, 256, BF16, p[0] + 1024, None) == ar.AR_ERR_ALIAS
    # norm_out overlapping residual_out; gamma inside an output.
    args = (_ptrs(p[:2]), 2, 4, 256, BF16, 0xA00000, 0xB00000, 1e-6)
    assert L.ar_residual_rmsnorm(*args, 0xC00000, 0xC00000 + 512, None) == ar.AR_ERR_ALIAS
    assert L.ar_residual_rmsnorm(_ptrs(p[:2]), 2, 4, 256, BF16, 0xA00000, 0xC00000 + 256, 1e-6,
                                 0xC00000, 0xD00000, None) == ar.AR_ERR_ALIAS
    # Bad eps, bad dtype, bad H for the norm.
    assert L.ar_residual_rmsnorm(_ptrs(p[:2]), 2, 4, 256, BF16, 0xA00000, 0xB00000, -1e-6,
                                 0xC00000, 0xD00000, None) == ar.AR_ERR_INVALID_ARG
    assert L.ar_residual_rmsnorm(_ptrs(p[:2]), 2, 4, 256, BF16, 0xA00000, 0xB00000,
                                 float("inf"), 0xC00000, 0xD00000, None) == ar.AR_ERR_INVALID_ARG
    assert L.ar_sum(_ptrs(p[:2]), 2, 4, 256, 9, out, None) == ar.AR_ERR_INVALID_ARG
    assert L.ar_residual_rmsnorm(_ptrs(p[:2]), 2, 4, 260, BF16, 0xA00000, 0xB00000, 1e-6,
                                 0xC00000, 0xD00000, None) == ar.AR_ERR_UNSUPPORTED
    # A with_config call with a malformed shape or a null shape.
    bad = ar.LaunchConfig(threads_per_block=100, vecs_per_thread=1, lanes_per_row=0,
                          rows_per_block=0, grid=1, flat=1)
    assert L.ar_sum_with_config(_ptrs(p[:2]), 2, 4, 256, BF16, out, None,
                                ctypes.byref(bad)) == ar.AR_ERR_INVALID_ARG
    assert L.ar_sum_with_config(_ptrs(p[:2]), 2, 4, 256, BF16, out, None,
                                None) == ar.AR_ERR_INVALID_ARG
    # Fixed rank batches: never for the sum, and for the norm only where they are built.
    sum_rat = ar.LaunchConfig(threads_per_block=64, vecs_per_thread=1, lanes_per_row=0,
                              rows_per_block=0, grid=1, flat=1, nt_store=1, ranks_per_batch=1)
    assert L.ar_sum_with_config(_ptrs(p[:2]), 2, 4, 256, BF16, out, None,
                                ctypes.byref(sum_rat)) == ar.AR_ERR_INVALID_ARG
    nargs = (_ptrs(p[:2]), 2, 4, 256, BF16, 0xA00000, 0xB00000, 1e-6, 0xC00000, 0xD00000, None)
    for vpt, lanes, nt, n in ((8, 64, 1, 1), (2, 64, 0, 1), (2, 64, 1, 3), (1, 64, 1, 1),
                              (2, 64, 1, 1), (2, 64, 1, 2), (2, 64, 1, 4), (4, 64, 1, 2),
                              (2, 64, 1, -1), (2, 64, 1, 8)):   # W = 2: 2 vectors take none
        cfg = ar.LaunchConfig(threads_per_block=64, vecs_per_thread=vpt, lanes_per_row=lanes,
                              rows_per_block=1, grid=4, flat=0, nt_store=nt, ranks_per_batch=n)
        assert L.ar_residual_rmsnorm_with_config(*nargs, ctypes.byref(cfg)) == \
            ar.AR_ERR_INVALID_ARG, (vpt, nt, n)
    many = (_ptrs(p[:16] * 2), 32, 4, 256, BF16, 0xA00000, 0xB00000, 1e-6, 0xC00000, 0xD00000,
            None)
    for vpt, nt, n in ((2, 1, 1), (2, 1, 4), (1, 1, 4), (4, 1, 2), (2, 0, 2), (1, 0, 2)):
        cfg = ar.LaunchConfig(threads_per_block=64, vecs_per_thread=vpt, lanes_per_row=64,
                              rows_per_block=1, grid=4, flat=0, nt_store=nt, ranks_per_batch=n)
        assert L.ar_residual_rmsnorm_with_config(*many, ctypes.byref(cfg)) == \
            ar.AR_ERR_INVALID_ARG, (vpt, nt, n)
    eight = (_ptrs(p[:8]), 8, 4, 256, BF16, 0xA00000, 0xB00000, 1e-6, 0xC00000, 0xD00000, None)
    for vpt, n in ((1, 2), (1, 4), (4, 4), (4, 2)):
        cfg = ar.LaunchConfig(threads_per_block=64, vecs_per_thread=vpt, lanes_per_row=64,
                              rows_per_block=1, grid=4, flat=0, nt_store=1, ranks_per_batch=n)
        assert L.ar_residual_rmsnorm_with_config(*eight, ctypes.byref(cfg)) == \
            ar.AR_ERR_INVALID_ARG, (vpt, n)


def test_zero_rows_returns_ok_without_device(L):
    """M = 0 is accepted before any device access (null pointers allowed for empty tensors)."""
    assert L.ar_sum(None, 2, 0, 256, BF16, None, None) == ar.AR_OK
    assert L.ar_residual_rmsnorm(None, 2, 0, 256, BF16, None, None, 1e-6, None, None,
                                 None) == ar.AR_OK


def test_unfused_and_rmsnorm_validation(L):
    """The two-kernel path takes any row width but the same world sizes, pointers and alias
    rules; the stand-alone RMSNorm rejects null, misaligned and overlapping buffers."""
    p = [0x10000 * (i + 1) for i in range(16)]
    args = (2, 4, 7170, BF16, 0xA00000, 0xB00000, 1e-6, 0xC00000, 0xD00000, None)
    assert L.ar_residual_rmsnorm_unfused(_ptrs(p[:12]), 12, 4, 7170, BF16, 0xA00000, 0xB00000,
                                         1e-6, 0xC00000, 0xD00000, None) == ar.AR_ERR_UNSUPPORTED
    assert L.ar_residual_rmsnorm_unfused(None, *args) == ar.AR_ERR_INVALID_ARG
    assert L.ar_residual_rmsnorm_unfused(_ptrs([p[0] + 2, p[1]]), *args) == ar.AR_ERR_MISALIGNED
    assert L.ar_residual_rmsnorm_unfused(_ptrs(p[:2]), 2, 4, 7170, BF16, 0xA00000, 0xB00000,
                                         -1.0, 0xC00000, 0xD00000, None) == ar.AR_ERR_INVALID_ARG
    # norm_out overlapping residual_out.
    assert L.ar_residual_rmsnorm_unfused(_ptrs(p[:2]), 2, 4, 7170, BF16, 0xA00000, 0xB00000,
                                         1e-6, 0xC00000, 0xC00000 + 4096, None) == ar.AR_ERR_ALIAS
    assert L.ar_residual_rmsnorm_unfused(None, 2, 0, 7170, BF16, None, None, 1e-6, None, None,
                                         None) == ar.AR_OK
    # Stand-alone RMSNorm.
    x, g, y = 0x100000, 0x200000, 0x300000
    assert L.ar_rmsnorm(None, 4, 7, BF16, g, 1e-6, y, None) == ar.AR_ERR_INVALID_ARG
    assert L.ar_rmsnorm(x, 4, 0, BF16, g, 1e-6, y, None) == ar.AR_ERR_INVALID_ARG
    assert L.ar_rmsnorm(x, 4, 7, 5, g, 1e-6, y, None) == ar.AR_ERR_INVALID_ARG
    assert L.ar_rmsnorm(x, 4, 7, BF16, g, float("nan"), y, None) == ar.AR_ERR_INVALID_ARG
    assert L.ar_rmsnorm(x + 2, 4, 7, BF16, g, 1e-6, y, None) == ar.AR_ERR_MISALIGNED
    assert L.ar_rmsnorm(x, 4, 7, BF16, g + 4, 1e-6, y, None) == ar.AR_ERR_MISALIGNED
    assert L.ar_rmsnorm(x, 4, 7, BF16, g, 1e-6, x + 16, None) == ar.AR_ERR_ALIAS
    assert L.ar_rmsnorm(x, 4, 7, BF16, y + 16, 1e-6, y, None) == ar.AR_ERR_ALIAS
    assert L.ar_rmsnorm(x, 1 << 40, 1 << 30, BF16, g, 1e-6, y, None) == ar.AR_ERR_UNSUPPORTED
    assert L.ar_rmsnorm(None, 0, 7, BF16, None, 1e-6, None, None) == ar.AR_OK


def test_probe_library_exports_and_rejects():
    """The benchmark's probes (bench_probes/ar_probe.h) are a library of their own; it exports
    its two functions and rejects malformed calls before any device access."""
    import os
    import re
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    path = os.path.join(root, "all_reduce_residual_amd", "libar_probe.so")
    with open(os.path.join(root, "all_reduce_residual_amd", "bench_probes", "ar_probe.h")) as f:
        text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
    assert re.findall(r"^\s*int\s+(ar_\w+)\s*\(", text, flags=re.M) == ["ar_probe_stream",
                                                                     "ar_probe_phases"]
    P = ctypes.CDLL(path)
    fn = P.ar_probe_stream
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p,
                   ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    fn.restype = ctypes.c_int
    p = _ptrs([0x10000 * (i + 1) for i in range(9)])
    assert fn(p, 7, 1, 64, 0x900000, 0xA00000, 64, None) == 1      # stream count
    assert fn(p, 9, 3, 64, 0x900000, 0xA00000, 64, None) == 1
    assert fn(p, 9, 2, 64, 0x900000, 0xA00000, 100, None) == 1     # threads
    assert fn(p, 9, 2, 64, 0x900008, 0xA00000, 64, None) == 1      # misaligned output
    assert fn(None, 9, 2, 64, 0x900000, 0xA00000, 64, None) == 1
    assert fn(p, 9, 2, 0, 0x900000, 0xA00000, 64, None) == 0       # nothing to do
    ph = P.ar_probe_phases
    ph.argtypes = [ctypes.c_int] * 8 + [ctypes.POINTER(ctypes.c_double)]
    ph.restype = ctypes.c_int
    out = (ctypes.c_double * 11)()
    assert ph(0, 8, 1, 7168, 64, 2, 6, 0, out) == 1      # grid does not cover the row
    assert ph(1, 8, 2, 7168, 448, 2, 1, 0, out) == 1     # one block per row: grid = M
    assert ph(1, 8, 1, 7168, 256, 2, 1, 0, out) == 1     # 256 x 2 vectors < 896
    assert ph(2, 8, 1, 7168, 64, 1, 14, 13, out) == 1    # segments x threads < 896
    assert ph(2, 8, 1, 7168, 64, 1, 13, 14, out) == 1    # grid != M x segments
    assert ph(1, 3, 1, 7168, 448, 2, 1, 0, out) == 1     # world size
    assert ph(4, 8, 1, 7168, 448, 2, 1, 0, out) == 1     # kind
    assert ph(1, 8, 1, 7168, 448, 2, 1, 0, None) == 1


def test_split_workspace_bytes(L):
    assert L.ar_split_workspace_bytes(0) == 0
    assert L.ar_split_workspace_bytes(1) == ar.SPLIT_SLOTS * 8
    assert L.ar_split_workspace_bytes(2048) == 2048 * ar.SPLIT_SLOTS * 8
    assert L.ar_split_workspace_bytes(-1) == -1
    assert L.ar_split_workspace_bytes(1 << 41) == -1


def test_split_config_invariants():
    """Planned split shapes are well formed: whole waves, one or two vectors per thread, 2..64
    segments covering the row exactly once, and a grid of M * S blocks that fits an int; no split
    once rows alone fill the GPU."""
    for W, M, H, dt in itertools.product(ar.SUPPORTED_W, [1, 2, 3, 8, 31, 64, 128, 200, 256, 512,
                                                           4096],
                                         [8, 256, 1024, 1032, 4096, 7168, 8192, 16384, 65536],
                                         [BF16, FP16, FP32]):
        if ar.ar_supports(RMS, W, M, H, dt) != ar.AR_OK:
            continue
        c = ar.ar_split_config(W, M, H, dt, 256)
        if c["segments"] == 0:
            assert c == {"threads_per_block": 0, "vecs_per_thread": 0, "segments": 0,
                         "max_polls": 0}
            continue
        V = H // (4 if dt == FP32 else 8)
        t, v, S = c["threads_per_block"], c["vecs_per_thread"], c["segments"]
        assert t % 64 == 0 and 64 <= t <= 1024 and v in (1, 2), c
        assert 2 <= S <= ar.SPLIT_SLOTS and S == -(-V // (t * v)), (W, M, H, c)
        assert (S - 1) * t * v < V <= S * t * v
        assert M * S < 2 ** 31 and c["max_polls"] > 0
    assert ar.ar_split_config(8, 4096, 7168, BF16, 256)["segments"] == 0
    # Two segments: rows >= 192 KiB up to a full grid, rows >= 112 KiB (W = 8 at H = 7168) while
    # an eighth of the CUs stays free; W = 4 rows never.
    assert ar.ar_split_config(8, 112, 7168, BF16, 256)["segments"] == 2
    assert ar.ar_split_config(8, 96, 8192, FP16, 256)["segments"] == 2
    assert ar.ar_split_config(8, 128, 7168, BF16, 256)["segments"] == 0
    assert ar.ar_split_config(16, 128, 7168, BF16, 256)["segments"] == 2
    assert ar.ar_split_config(4, 96, 8192, BF16, 256)["segments"] == 0
    assert ar.ar_split_config(8, 1, 7168, BF16, 256)["segments"] >= 2
    with pytest.raises(ar.ArError) as e:
        ar.ar_split_config(12, 4, 7168, BF16, 256)
    assert e.value.status == ar.AR_ERR_UNSUPPORTED
    with pytest.raises(ar.ArError) as e:
        ar.ar_split_config(8, 4, 7170, BF16, 256)
    assert e.value.status == ar.AR_ERR_UNSUPPORTED


def test_split_validation_rejects_before_device_access(L):
    """Workspace and split-shape checks reject before any device access (fake pointers)."""
    p = [0x10000 * (i + 1) for i in range(16)]
    M, H = 4, 7168
    res, gam, ro, no = 0x1000000, 0x2000000, 0x3000000, 0x4000000
    ws = 0x5000000
    need = L.ar_split_workspace_bytes(M)

    def ws_call(workspace, nbytes, cfg=None, ins=p[:8], W=8, r_out=ro, n_out=no):
        if cfg is None:
            return L.ar_residual_rmsnorm_ws(_ptrs(ins), W, M, H, BF16, res, gam, 1e-6, r_out,
                                            n_out, workspace, nbytes, None)
        return L.ar_residual_rmsnorm_split_with_config(_ptrs(ins), W, M, H, BF16, res, gam, 1e-6,
                                                       r_out, n_out, workspace, nbytes, None,
                                                       ctypes.byref(cfg))

    good = ar.SplitConfig(threads_per_block=64, vecs_per_thread=1, segments=14, max_polls=100)
    assert ws_call(None, need) == ar.AR_ERR_INVALID_ARG
    assert ws_call(ws, need - 8) == ar.AR_ERR_INVALID_ARG
    assert ws_call(ws, -1) == ar.AR_ERR_INVALID_ARG
    assert ws_call(ws + 8, need) == ar.AR_ERR_MISALIGNED
    assert ws_call(ro + 1024, need) == ar.AR_ERR_ALIAS                 # inside residual_out
    assert ws_call(p[3] + 512, need) == ar.AR_ERR_ALIAS                # inside a partial
    assert ws_call(gam - 256, need) == ar.AR_ERR_ALIAS                 # over gamma
    # Malformed split shapes.
    for bad in (dict(threads_per_block=96, vecs_per_thread=1, segments=10),
                dict(threads_per_block=64, vecs_per_thread=4, segments=4),
                dict(threads_per_block=64, vecs_per_thread=1, segments=13),
                dict(threads_per_block=2048, vecs_per_thread=1, segments=1)):
        cfg = ar.SplitConfig(max_polls=1, **bad)
        assert ws_call(ws, need, cfg) == ar.AR_ERR_INVALID_ARG, bad
    assert L.ar_residual_rmsnorm_split_with_config(_ptrs(p[:8]), 8, M, H, BF16, res, gam, 1e-6,
                                                   ro, no, ws, need, None,
                                                   None) == ar.AR_ERR_INVALID_ARG
    # More than 64 segments (H = 65536 bf16 at 64 x 1 vectors per block: 128).
    cfg = ar.SplitConfig(threads_per_block=64, vecs_per_thread=1, segments=128, max_polls=1)
    assert L.ar_residual_rmsnorm_split_with_config(
        _ptrs(p[:8]), 8, M, 65536, BF16, res, gam, 1e-6, ro, no, ws, need, None,
        ctypes.byref(cfg)) == ar.AR_ERR_INVALID_ARG
    # Split launches take up to 65535 rows (their grid is S x M blocks).
    big = 65536
    q = [(i + 1) << 32 for i in range(8)]                 # 4 GiB apart: no overlaps
    assert L.ar_residual_rmsnorm_split_with_config(
        _ptrs(q), 8, big, H, BF16, 20 << 32, 21 << 32, 1e-6, 22 << 32, 23 << 32, 24 << 32,
        L.ar_split_workspace_bytes(big), None, ctypes.byref(good)) == ar.AR_ERR_UNSUPPORTED
    # The explicit split refuses outputs that alias the residual or an input.
    assert ws_call(ws, need, good, r_out=res) == ar.AR_ERR_ALIAS
    assert ws_call(ws, need, good, n_out=p[2]) == ar.AR_ERR_ALIAS
    # Ordinary norm validation still applies (world size 12, bad eps).
    assert ws_call(ws, need, ins=p[:12], W=12) == ar.AR_ERR_UNSUPPORTED
    assert L.ar_residual_rmsnorm_ws(None, 8, 0, H, BF16, None, None, 1e-6, None, None, None, 0,
                                    None) == ar.AR_OK
    # Workspace clearing: null, misaligned, not a multiple of 8; zero bytes is a no-op.
    assert L.ar_workspace_clear(None, 64, None) == ar.AR_ERR_INVALID_ARG
    assert L.ar_workspace_clear(ws + 8, 64, None) == ar.AR_ERR_MISALIGNED
    assert L.ar_workspace_clear(ws, 12, None) == ar.AR_ERR_INVALID_ARG
    assert L.ar_workspace_clear(ws, 0, None) == ar.AR_OK


def test_noalloc_validation_rejects_before_device_access(L):
    """The no-allocation form validates like ar_residual_rmsnorm and rejects more rows than its
    device array holds, all before any device access (fake pointers); M = 0 is a no-op."""
    p = [0x10000 * (i + 1) for i in range(16)]
    H = 7168
    res, gam, ro, no = 0x1000000, 0x2000000, 0x3000000, 0x4000000

    def call(M, ins=p[:8], W=8, eps=1e-6, r_out=ro, n_out=no):
        return L.ar_residual_rmsnorm_noalloc(_ptrs(ins), W, M, H, BF16, res, gam, eps, r_out,
                                             n_out, None)

    assert ar.NOALLOC_MAX_ROWS == 512
    assert call(ar.NOALLOC_MAX_ROWS + 1) == ar.AR_ERR_UNSUPPORTED
    assert call(1 << 20) == ar.AR_ERR_UNSUPPORTED
    assert call(4, ins=p[:12], W=12) == ar.AR_ERR_UNSUPPORTED
    assert call(4, eps=-1.0) == ar.AR_ERR_INVALID_ARG
    assert call(4, n_out=ro) == ar.AR_ERR_ALIAS
    assert call(4, r_out=ro + 8) == ar.AR_ERR_MISALIGNED
    assert L.ar_residual_rmsnorm_noalloc(None, 8, 0, H, BF16, None, None, 1e-6, None, None,
                                         None) == ar.AR_OK
