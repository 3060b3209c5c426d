"""Boundary behaviour of the C ABI on the GPU: rejections write nothing, outputs stay inside
their buffers, inputs are preserved, results are deterministic, in-place aliasing works, and a
captured hipGraph replays to the same results as eager calls (the graph-replay correctness and
input-preservation checks and the world-size-12 rejection described in the vLLM pull request
"[Perf] Tune FlashInfer all-reduce selection on SM103", Tests).
"""
import numpy as np
import pytest
import torch

import all_reduce_residual_amd as ar
import synth
from gpu_util import assert_bit_exact, assert_norm_close, dev, host_np

pytestmark = pytest.mark.gpu

CANARY = 0x5A5A


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    ar.lib()


def _guarded(M, H, dtype, guard=4096):
    """[M, H] view in the middle of a buffer whose guard bands hold a canary pattern."""
    n = M * H
    buf = torch.full((guard + n + guard,), CANARY, dtype=torch.int16, device="cuda")
    buf = buf.view(synth.TORCH_DTYPES[dtype]) if dtype != "fp32" else \
        torch.full((guard + n + guard,), 1.2345e-7, dtype=torch.float32, device="cuda")
    return buf, buf[guard:guard + n].view(M, H), guard


def _guards_intact(buf, guard, n):
    b = host_np(buf.cpu())
    head, tail = b[:guard], b[guard + n:]
    if b.dtype == np.float32:
        return (head == np.float32(1.2345e-7)).all() and (tail == np.float32(1.2345e-7)).all()
    return (head == CANARY).all() and (tail == CANARY).all()


def _inputs(W, M, H, dtype, seed):
    parts, res, gam = synth.custom(W, M, H, dtype, seed)
    return parts, res, gam, [dev(p) for p in parts], dev(res), dev(gam)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_outputs_stay_in_bounds(oracle_mod, dtype):
    W, M, H = 8, 37, 1016 if dtype == "bf16" else 1012
    parts, res, gam, dp, dr, dg = _inputs(W, M, H, dtype, 1)
    b1, ro, g = _guarded(M, H, dtype)
    b2, no, _ = _guarded(M, H, dtype)
    b3, out, _ = _guarded(M, H, dtype)
    ar.ar_residual_rmsnorm(dp, dr, dg, 1e-6, ro, no)
    ar.ar_sum(dp, out)
    torch.cuda.synchronize()
    for b in (b1, b2, b3):
        assert _guards_intact(b, g, M * H)
    want_ro, want_no = oracle_mod.ar_residual_rmsnorm([host_np(p) for p in parts], host_np(res),
                                                      gam.numpy(), 1e-6, dtype)
    assert_bit_exact(host_np(ro.cpu()), want_ro, dtype, "residual_out")
    assert_norm_close(host_np(no.cpu()), want_no, dtype)


def test_sum_tail_stays_in_bounds():
    M, H = 3, 13
    parts, _, _, dp, _, _ = _inputs(4, M, H, "bf16", 2)
    b, out, g = _guarded(M, H, "bf16")
    ar.ar_sum(dp, out)
    torch.cuda.synchronize()
    assert _guards_intact(b, g, M * H)


def test_inputs_preserved_and_deterministic():
    W, M, H = 8, 64, 7168
    _, _, _, dp, dr, dg = _inputs(W, M, H, "bf16", 3)
    before = [t.clone() for t in dp + [dr, dg]]
    ro, no, out = torch.empty_like(dr), torch.empty_like(dr), torch.empty_like(dr)
    ar.ar_residual_rmsnorm(dp, dr, dg, 1e-6, ro, no)
    ar.ar_sum(dp, out)
    first = (ro.clone(), no.clone(), out.clone())
    for _ in range(100):
        ar.ar_residual_rmsnorm(dp, dr, dg, 1e-6, ro, no)
        ar.ar_sum(dp, out)
    torch.cuda.synchronize()
    for a, b in zip(before, dp + [dr, dg]):
        assert torch.equal(a.view(torch.int16) if a.dtype != torch.float32 else a,
                           b.view(torch.int16) if b.dtype != torch.float32 else b)
    for a, b in zip(first, (ro, no, out)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_in_place_aliasing(oracle_mod):
    """out may be one of the inputs; residual_out may be the residual; norm_out may be an
    input -- exact aliases only."""
    W, M, H = 4, 9, 2048
    parts, res, gam, dp, dr, dg = _inputs(W, M, H, "bf16", 4)
    want_sum = oracle_mod.ar_sum([host_np(p) for p in parts], "bf16")
    want_ro, want_no = oracle_mod.ar_residual_rmsnorm([host_np(p) for p in parts], host_np(res),
                                                      gam.numpy(), 1e-6, "bf16")
    a = [t.clone() for t in dp]
    ar.ar_sum(a, a[2])
    torch.cuda.synchronize()
    assert_bit_exact(host_np(a[2].cpu()), want_sum, "bf16", "out in place")
    b = [t.clone() for t in dp]
    r = dr.clone()
    ar.ar_residual_rmsnorm(b, r, dg, 1e-6, r, b[0])
    torch.cuda.synchronize()
    assert_bit_exact(host_np(r.cpu()), want_ro, "bf16", "residual_out in place")
    assert_norm_close(host_np(b[0].cpu()), want_no, "bf16")


def _expect_status(status, fn):
    with pytest.raises(ar.ArError) as e:
        fn()
    assert e.value.status == status, (e.value.status, str(e.value))


def test_rejections_write_nothing():
    M, H = 8, 256
    _, _, _, dp, dr, dg = _inputs(16, M, H, "bf16", 5)
    ro = torch.full((M, H), CANARY, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    no = torch.full((M, H), CANARY, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    out = torch.full((M, H), CANARY, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    # World size 12: rejected at run time (the pages' unsupported world size).
    _expect_status(ar.AR_ERR_UNSUPPORTED, lambda: ar.ar_sum(dp[:12], out))
    _expect_status(ar.AR_ERR_UNSUPPORTED,
                   lambda: ar.ar_residual_rmsnorm(dp[:12], dr, dg, 1e-6, ro, no))
    _expect_status(ar.AR_ERR_UNSUPPORTED, lambda: ar.ar_sum(dp[:3], out))
    # Bad eps.
    _expect_status(ar.AR_ERR_INVALID_ARG,
                   lambda: ar.ar_residual_rmsnorm(dp[:2], dr, dg, -1.0, ro, no))
    _expect_status(ar.AR_ERR_INVALID_ARG,
                   lambda: ar.ar_residual_rmsnorm(dp[:2], dr, dg, float("nan"), ro, no))
    # norm_out == residual_out.
    _expect_status(ar.AR_ERR_ALIAS, lambda: ar.ar_residual_rmsnorm(dp[:2], dr, dg, 1e-6, ro, ro))
    # Partial overlap of an output with an input.
    flat = torch.empty(M * H * 2, dtype=torch.bfloat16, device="cuda")
    in0 = flat[:M * H].view(M, H)
    shifted = flat[64:64 + M * H].view(M, H)
    _expect_status(ar.AR_ERR_ALIAS, lambda: ar.ar_sum([in0, dp[1]], shifted))
    # Misaligned (2-byte offset) tensor.
    mis = flat[1:1 + M * H].view(M, H)
    _expect_status(ar.AR_ERR_MISALIGNED, lambda: ar.ar_sum([mis, dp[1]], out))
    # A malformed launch shape.
    bad = dict(threads_per_block=96, vecs_per_thread=1, lanes_per_row=32, rows_per_block=3,
               grid=1, flat=0)
    _expect_status(ar.AR_ERR_INVALID_ARG,
                   lambda: ar.ar_residual_rmsnorm(dp[:2], dr, dg, 1e-6, ro, no, config=bad))
    short = dict(threads_per_block=64, vecs_per_thread=1, lanes_per_row=16, rows_per_block=4,
                 grid=1, flat=0)   # 16 lanes x 1 vector cannot cover a 32-vector row
    _expect_status(ar.AR_ERR_INVALID_ARG,
                   lambda: ar.ar_residual_rmsnorm(dp[:2], dr, dg, 1e-6, ro, no, config=short))
    torch.cuda.synchronize()
    for t in (ro, no, out):
        assert (t.view(torch.int16) == CANARY).all()


def test_zero_rows_is_a_no_op():
    H = 512
    z = [torch.empty(0, H, dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    g = torch.ones(H, dtype=torch.float32, device="cuda")
    ar.ar_sum(z, torch.empty(0, H, dtype=torch.bfloat16, device="cuda"))
    ar.ar_residual_rmsnorm(z, z[0], g, 1e-6, torch.empty(0, H, dtype=torch.bfloat16, device="cuda"),
                           torch.empty(0, H, dtype=torch.bfloat16, device="cuda"))
    torch.cuda.synchronize()


def test_graph_replay_matches_eager(oracle_mod):
    """Capture one call of each pattern in a hipGraph, then replay it several times with new
    input contents written into the same buffers (and eager work in between); every replay
    must equal the oracle for the inputs current at that replay."""
    W, M, H, dtype = 8, 32, 7168, "bf16"
    parts, res, gam, dp, dr, dg = _inputs(W, M, H, dtype, 6)
    ro, no, out = torch.empty_like(dr), torch.empty_like(dr), torch.empty_like(dr)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ar.ar_residual_rmsnorm(dp, dr, dg, 1e-6, ro, no)
        ar.ar_sum(dp, out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ar.ar_residual_rmsnorm(dp, dr, dg, 1e-6, ro, no)
        ar.ar_sum(dp, out)
    for rep in range(4):
        p2, r2, _ = synth.custom(W, M, H, dtype, seed=100 + rep)
        for d, h in zip(dp + [dr], p2 + [r2]):
            d.copy_(h)
        # Unrelated eager work between replays.
        scratch = torch.empty_like(dr)
        ar.ar_sum(dp[:2], scratch)
        graph.replay()
        torch.cuda.synchronize()
        hp = [host_np(p) for p in p2]
        want_ro, want_no = oracle_mod.ar_residual_rmsnorm(hp, host_np(r2), gam.numpy(), 1e-6,
                                                          dtype)
        assert_bit_exact(host_np(ro.cpu()), want_ro, dtype, "replay %d residual_out" % rep)
        assert_norm_close(host_np(no.cpu()), want_no, dtype, "replay %d norm_out" % rep)
        assert_bit_exact(host_np(out.cpu()), oracle_mod.ar_sum(hp, dtype), dtype,
                         "replay %d out" % rep)
        # Inputs untouched by the replay.
        assert torch.equal(dr.cpu().view(torch.int16), r2.view(torch.int16))


def test_graph_replay_of_exchange_gather_and_fallback(oracle_mod):
    """The Lamport exchange (three rounds of W pushes + the polling consumer, so that replays keep
    the buffer rotation), the all-gather of a two-shot round and the two-kernel path, captured
    once and replayed with new inputs and eager work in between: every replay equals the oracle,
    and the exchange's status word stays clear (each round finds its buffer emptied by the pushes
    of the round before)."""
    W, M, H, dtype = 8, 24, 7168, "bf16"
    parts, res, gam, dp, dr, dg = _inputs(W, M, H, dtype, 21)
    rbuf = torch.empty((ar.LAMPORT_BUFFERS, W, M, H), dtype=torch.bfloat16, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    ar.ar_lamport_arm(rbuf)
    lro, lno = torch.empty_like(dr), torch.empty_like(dr)
    # Two-shot gather of the rank slices of `gsrc` into `gout`.
    gsrc = torch.empty_like(dr)
    gout = torch.empty_like(dr)
    slices = []
    for j in range(W):
        b, c = ar.ar_row_partition(W, M, j)
        slices.append(gsrc[b:b + c])
    # Two-kernel path on an odd width.
    Hu = 7170
    up, ur, ug = synth.custom(4, M, Hu, dtype, seed=22)
    dup, dur, dug = [dev(p) for p in up], dev(ur), dev(ug)
    uro, uno = torch.empty_like(dur), torch.empty_like(dur)

    def calls():
        for rnd in range(ar.LAMPORT_BUFFERS):
            for r in range(W):
                ar.ar_lamport_push(dp[r], r, rbuf, rnd)
            ar.ar_lamport_residual_rmsnorm(rbuf, rnd, dr, dg, 1e-6, lro, lno, status)
        ar.ar_all_gather(slices, gout)
        ar.ar_residual_rmsnorm_unfused(dup, dur, dug, 1e-6, uro, uno)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        calls()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    for rep in range(3):
        p2, r2, _ = synth.custom(W, M, H, dtype, seed=200 + rep)
        for d, h in zip(dp + [dr], p2 + [r2]):
            d.copy_(h)
        g2 = synth.custom(1, M, H, dtype, seed=300 + rep)[0][0]
        gsrc.copy_(g2)
        u2, ur2, _ = synth.custom(4, M, Hu, dtype, seed=400 + rep)
        for d, h in zip(dup + [dur], u2 + [ur2]):
            d.copy_(h)
        ar.ar_sum(dp[:2], torch.empty_like(dr))          # unrelated eager work
        graph.replay()
        torch.cuda.synchronize()
        assert int(status.item()) == 0, "replay %d: a poll timed out" % rep
        want_ro, want_no = oracle_mod.ar_residual_rmsnorm(
            [host_np(p) for p in p2], host_np(r2), gam.numpy(), 1e-6, dtype)
        assert_bit_exact(host_np(lro.cpu()), want_ro, dtype, "replay %d lamport residual_out" % rep)
        assert_norm_close(host_np(lno.cpu()), want_no, dtype, "replay %d lamport norm_out" % rep)
        assert_bit_exact(host_np(gout.cpu()), host_np(g2), dtype, "replay %d gather" % rep)
        want_ro, want_no = oracle_mod.ar_residual_rmsnorm(
            [host_np(p) for p in u2], host_np(ur2), ug.numpy(), 1e-6, dtype)
        assert_bit_exact(host_np(uro.cpu()), want_ro, dtype, "replay %d unfused residual_out" % rep)
        assert_norm_close(host_np(uno.cpu()), want_no, dtype, "replay %d unfused norm_out" % rep)
    # The last round (2) emptied buffer 0 for the next replay's round 0.
    assert bool((rbuf[0].view(torch.int16) == -1).all())


def test_device_facts():
    cu = ar.ar_device_cu_count()
    print("compute units:", cu, torch.cuda.get_device_name(0))
    assert cu > 0
    assert ar.ar_launch_config(1, 8, 2048, 7168, ar.DTYPE_BF16) == \
        ar.ar_launch_config(1, 8, 2048, 7168, ar.DTYPE_BF16, cu_count=cu)
