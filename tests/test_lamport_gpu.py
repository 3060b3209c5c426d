"""Lamport-style one-shot exchange on the GPU: producers push their partials into their slots
of this round's receive buffer (and empty their slots of the next one), the consumer polls and
reduces exactly like the plain entry points.  Results are compared with the oracle (bit-identical
out/residual_out, norm_out within 1 ulp); after round k the buffer of round k + 1 is empty and
the buffer of round k holds every partial (an all-ones element with its lowest bit cleared).
Every wait is bounded, and the one test that exercises a timeout forces it from the host with a
spin limit of 4 polls (the kernel still finishes).
"""
import numpy as np
import pytest
import torch

import all_reduce_residual_amd as ar
import synth
from gpu_util import assert_bit_exact, assert_norm_close, dev, host_np

pytestmark = pytest.mark.gpu

NBUF = ar.LAMPORT_BUFFERS


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    ar.lib()


def _int_view(t):
    return t.view(torch.int32 if t.dtype == torch.float32 else torch.int16)


def _empty(t):
    return bool((_int_view(t) == -1).all())


def _new_rbuf(W, M, H, tdt):
    rbuf = torch.empty((NBUF, W, M, H), dtype=tdt, device="cuda")
    ar.ar_lamport_arm(rbuf)
    return rbuf


def _delivered(p):
    """What a producer stores for partial p: all-ones elements with their lowest bit cleared."""
    iv = _int_view(p.contiguous()).clone()
    iv[iv == -1] = -2
    return iv


def check_round_state(rbuf, rnd, d_parts):
    """After round rnd: the next round's buffer is empty and this round's holds every partial."""
    assert _empty(rbuf[(rnd + 1) % NBUF]), "round %d: next buffer not empty" % rnd
    for r, p in enumerate(d_parts):
        assert torch.equal(_int_view(rbuf[rnd % NBUF, r]), _delivered(p)), \
            "round %d: slot %d does not hold the partial" % (rnd, r)


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("W", [2, 8, 16])
def test_sequential_round(oracle_mod, dtype, W):
    M, H = 9, 1024
    parts, res, gam = synth.custom(W, M, H, dtype, seed=W)
    tdt = synth.TORCH_DTYPES[dtype]
    d_parts = [dev(p) for p in parts]
    hp = [host_np(p) for p in parts]
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    rbuf = _new_rbuf(W, M, H, tdt)
    for r, p in enumerate(d_parts):
        ar.ar_lamport_push(p, r, rbuf, 0)
    out = torch.empty_like(d_parts[0])
    ar.ar_lamport_sum(rbuf, 0, out, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    check_round_state(rbuf, 0, d_parts)
    assert_bit_exact(host_np(out.cpu()), oracle_mod.ar_sum(hp, dtype), dtype, "lamport out")
    for r, p in enumerate(d_parts):
        ar.ar_lamport_push(p, r, rbuf, 1)
    d_res, d_gam = dev(res), dev(gam)
    ro, no = torch.empty_like(d_res), torch.empty_like(d_res)
    ar.ar_lamport_residual_rmsnorm(rbuf, 1, d_res, d_gam, 1e-6, ro, no, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    check_round_state(rbuf, 1, d_parts)
    want_ro, want_no = oracle_mod.ar_residual_rmsnorm(hp, host_np(res), gam.numpy(), 1e-6, dtype)
    assert_bit_exact(host_np(ro.cpu()), want_ro, dtype, "lamport residual_out")
    assert_norm_close(host_np(no.cpu()), want_no, dtype, "lamport norm_out")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("W", [4, 8, 16])
def test_smaller_polled_batches_beyond_one_row_per_cu(oracle_mod, dtype, W):
    """Two CUs' worth of rows and three more (H = 7168): both consumers poll smaller batches
    there (the sum two ranks at a time; the fused consumer two ranks with 2 vectors per thread,
    bf16, and one with 4, binary32).  Every row against the oracle."""
    M, H = 2 * ar.ar_device_cu_count() + 3, 7168
    print("case", W, M, H, dtype, flush=True)
    parts, res, gam = synth.custom(W, M, H, dtype, seed=W * 5 + M)
    tdt = synth.TORCH_DTYPES[dtype]
    d_parts = [dev(p) for p in parts]
    hp = [host_np(p) for p in parts]
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    rbuf = _new_rbuf(W, M, H, tdt)
    for r, p in enumerate(d_parts):
        ar.ar_lamport_push(p, r, rbuf, 0)
    out = torch.empty_like(d_parts[0])
    ar.ar_lamport_sum(rbuf, 0, out, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert_bit_exact(host_np(out.cpu()), oracle_mod.ar_sum(hp, dtype), dtype, "lamport out")
    for r, p in enumerate(d_parts):
        ar.ar_lamport_push(p, r, rbuf, 1)
    d_res, d_gam = dev(res), dev(gam)
    ro, no = torch.empty_like(d_res), torch.empty_like(d_res)
    ar.ar_lamport_residual_rmsnorm(rbuf, 1, d_res, d_gam, 1e-6, ro, no, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    check_round_state(rbuf, 1, d_parts)
    want_ro, want_no = oracle_mod.ar_residual_rmsnorm(hp, host_np(res), gam.numpy(), 1e-6, dtype)
    assert_bit_exact(host_np(ro.cpu()), want_ro, dtype, "lamport residual_out")
    assert_norm_close(host_np(no.cpu()), want_no, dtype, "lamport norm_out")


def test_rounds_rotate_through_three_buffers(oracle_mod):
    """Seven rounds (the rotation wraps twice) without re-arming: each push empties the next
    round's slots, so every round finds its buffer empty."""
    W, M, H, dtype = 8, 33, 7168, "bf16"
    tdt = synth.TORCH_DTYPES[dtype]
    rbuf = _new_rbuf(W, M, H, tdt)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    for rnd in range(7):
        parts, res, gam = synth.custom(W, M, H, dtype, seed=50 + rnd)
        d_parts = [dev(p) for p in parts]
        for r, p in enumerate(d_parts):
            ar.ar_lamport_push(p, r, rbuf, rnd)
        d_res, d_gam = dev(res), dev(gam)
        ro, no = torch.empty_like(d_res), torch.empty_like(d_res)
        ar.ar_lamport_residual_rmsnorm(rbuf, rnd, d_res, d_gam, 1e-6, ro, no, status)
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        check_round_state(rbuf, rnd, d_parts)
        want_ro, want_no = oracle_mod.ar_residual_rmsnorm([host_np(p) for p in parts],
                                                          host_np(res), gam.numpy(), 1e-6, dtype)
        assert_bit_exact(host_np(ro.cpu()), want_ro, dtype, "round %d residual_out" % rnd)
        assert_norm_close(host_np(no.cpu()), want_no, dtype, "round %d norm_out" % rnd)


@pytest.mark.parametrize("pattern", ["sum", "rms"])
def test_consumer_polls_while_producers_run(oracle_mod, pattern):
    """Producers on one stream, delayed by a sleep kernel, and the consumer on another, for four
    rounds.  The producer stream waits for the consumer's previous round (an event), as the
    ordering contract asks, and nothing else orders the two.  Streams share the GPU's few
    hardware queues, so each round enqueues the producers first: on separate queues the consumer
    starts and polls until the pushes land; on one queue the pushes simply run first."""
    W, M, H, dtype = 8, 8, 7168, "bf16"
    tdt = synth.TORCH_DTYPES[dtype]
    rbuf = _new_rbuf(W, M, H, tdt)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    consumer, producer = torch.cuda.Stream(), torch.cuda.Stream()
    for st in (consumer, producer):       # first use of a stream can take milliseconds
        with torch.cuda.stream(st):
            torch.zeros(1, device="cuda").add_(1)
    torch.cuda.synchronize()
    rounds = []
    for rnd in range(4):
        parts, res, gam = synth.custom(W, M, H, dtype, seed=77 + rnd)
        d_parts = [dev(p) for p in parts]
        d_res, d_gam = dev(res), dev(gam)
        out, ro, no = (torch.empty_like(d_res) for _ in range(3))
        torch.cuda.synchronize()          # inputs in place before either stream reads them
        producer.wait_stream(consumer)    # the consumer of round rnd - 1 is done
        with torch.cuda.stream(producer):
            torch.cuda._sleep(1 << 20)    # ~0.5 ms on the producer stream
        for r, p in enumerate(d_parts):
            ar.ar_lamport_push(p, r, rbuf, rnd, stream=producer)
        if pattern == "sum":
            ar.ar_lamport_sum(rbuf, rnd, out, status, spin_limit=1 << 20, stream=consumer)
        else:
            ar.ar_lamport_residual_rmsnorm(rbuf, rnd, d_res, d_gam, 1e-6, ro, no, status,
                                           spin_limit=1 << 20, stream=consumer)
        rounds.append((parts, res, gam, out, ro, no))
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    for rnd, (parts, res, gam, out, ro, no) in enumerate(rounds):
        hp = [host_np(p) for p in parts]
        if pattern == "sum":
            assert_bit_exact(host_np(out.cpu()), oracle_mod.ar_sum(hp, dtype), dtype,
                             "round %d out" % rnd)
        else:
            want_ro, want_no = oracle_mod.ar_residual_rmsnorm(hp, host_np(res), gam.numpy(),
                                                              1e-6, dtype)
            assert_bit_exact(host_np(ro.cpu()), want_ro, dtype, "round %d residual_out" % rnd)
            assert_norm_close(host_np(no.cpu()), want_no, dtype, "round %d norm_out" % rnd)
    check_round_state(rbuf, 3, [dev(p) for p in rounds[-1][0]])


def test_missing_producer_times_out_and_reports(oracle_mod):
    """One rank never pushes: with a spin limit of 4 polls the consumer gives up, sets the status
    bit and finishes (forced from the host; no unbounded wait exists).  Re-arming restores the
    exchange: the next round is exact."""
    W, M, H = 4, 2, 256
    parts, _, _ = synth.custom(W, M, H, "bf16", seed=5, with_norm=False)
    rbuf = _new_rbuf(W, M, H, torch.bfloat16)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    for r, p in enumerate(parts[:-1]):
        ar.ar_lamport_push(dev(p), r, rbuf, 0)
    out = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
    ar.ar_lamport_sum(rbuf, 0, out, status, spin_limit=4)
    torch.cuda.synchronize()
    assert int(status.item()) & 1 == 1
    ar.ar_lamport_arm(rbuf)
    torch.cuda.synchronize()
    assert _empty(rbuf)
    status.zero_()
    for r, p in enumerate(parts):
        ar.ar_lamport_push(dev(p), r, rbuf, 1)
    ar.ar_lamport_sum(rbuf, 1, out, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert_bit_exact(host_np(out.cpu()), oracle_mod.ar_sum([host_np(p) for p in parts], "bf16"),
                     "bf16", "after re-arm")


@pytest.mark.parametrize("pattern", ["sum", "rms"])
def test_missing_producer_times_out_with_smaller_polled_batches(oracle_mod, pattern):
    """The consumers' smaller polled batches (two CUs' worth of rows and three more) are bounded
    the same way: one rank never pushes, a spin limit of 4 polls, the status bit is set and the
    call finishes; after re-arming the next round is exact."""
    W, M, H = 8, 2 * ar.ar_device_cu_count() + 3, 7168
    print("case", pattern, W, M, H, flush=True)
    parts, res, gam = synth.custom(W, M, H, "bf16", seed=17 + M)
    rbuf = _new_rbuf(W, M, H, torch.bfloat16)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    d_parts = [dev(p) for p in parts]
    d_res, d_gam = dev(res), dev(gam)
    out = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
    ro, no = torch.empty_like(out), torch.empty_like(out)

    def consume(rnd, **kw):
        if pattern == "sum":
            ar.ar_lamport_sum(rbuf, rnd, out, status, **kw)
        else:
            ar.ar_lamport_residual_rmsnorm(rbuf, rnd, d_res, d_gam, 1e-6, ro, no, status, **kw)

    for r, p in enumerate(d_parts[:-1]):
        ar.ar_lamport_push(p, r, rbuf, 0)
    consume(0, spin_limit=4)
    torch.cuda.synchronize()
    assert int(status.item()) & 1 == 1
    ar.ar_lamport_arm(rbuf)
    status.zero_()
    for r, p in enumerate(d_parts):
        ar.ar_lamport_push(p, r, rbuf, 1)
    consume(1)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    hp = [host_np(p) for p in parts]
    if pattern == "sum":
        assert_bit_exact(host_np(out.cpu()), oracle_mod.ar_sum(hp, "bf16"), "bf16", "after re-arm")
    else:
        want_ro, want_no = oracle_mod.ar_residual_rmsnorm(hp, host_np(res), gam.numpy(), 1e-6,
                                                          "bf16")
        assert_bit_exact(host_np(ro.cpu()), want_ro, "bf16", "residual_out after re-arm")
        assert_norm_close(host_np(no.cpu()), want_no, "bf16", "norm_out after re-arm")


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_all_ones_input_is_not_mistaken_for_empty(oracle_mod, dtype):
    """A partial element that is all ones (a NaN) is delivered as a NaN with its lowest bit
    cleared; the reduction sees a NaN exactly where the oracle does, and nothing waits."""
    W, M, H = 4, 3, 64
    parts, res, gam = synth.custom(W, M, H, dtype, seed=11)
    iv = torch.int32 if dtype == "fp32" else torch.int16
    tdt = synth.TORCH_DTYPES[dtype]
    p0 = parts[1].view(iv).clone()
    p0[1, ::5] = -1
    parts[1] = p0.view(tdt)
    d_parts = [dev(p) for p in parts]
    rbuf = _new_rbuf(W, M, H, tdt)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    for r, p in enumerate(d_parts):
        ar.ar_lamport_push(p, r, rbuf, 0)
    out = torch.empty_like(d_parts[0])
    ar.ar_lamport_sum(rbuf, 0, out, status, spin_limit=64)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    check_round_state(rbuf, 0, d_parts)
    assert_bit_exact(host_np(out.cpu()), oracle_mod.ar_sum([host_np(p) for p in parts], dtype),
                     dtype, "out")


@pytest.mark.parametrize("name,M", [("wide_hidden", 2048), ("fp16_many_rank", 512),
                                    ("llama3_decode", 128)])
def test_workloads_through_the_exchange(oracle_mod, name, M):
    wl = synth.WORKLOADS[name]
    parts, res, gam = synth.inputs(wl, M)
    tdt = synth.TORCH_DTYPES[wl.dtype]
    rbuf = _new_rbuf(wl.W, M, wl.H, tdt)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    d_parts = [dev(p) for p in parts]
    for r, p in enumerate(d_parts):
        ar.ar_lamport_push(p, r, rbuf, 0)
    d_res, d_gam = dev(res), dev(gam)
    ro, no = torch.empty_like(d_res), torch.empty_like(d_res)
    ar.ar_lamport_residual_rmsnorm(rbuf, 0, d_res, d_gam, wl.eps, ro, no, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    check_round_state(rbuf, 0, d_parts)
    want_ro, want_no = oracle_mod.ar_residual_rmsnorm([host_np(p) for p in parts], host_np(res),
                                                      gam.numpy(), wl.eps, wl.dtype)
    assert_bit_exact(host_np(ro.cpu()), want_ro, wl.dtype, "residual_out")
    assert_norm_close(host_np(no.cpu()), want_no, wl.dtype)


@pytest.mark.parametrize("W,M,H,dtype", [(2, 2048, 4096, "bf16"), (1, 300, 4096, "fp16"),
                                         (4, 3, 65536, "bf16"), (8, 5, 32768, "bf16"),
                                         (16, 4, 32768, "fp16"), (64, 2, 16384, "bf16"),
                                         (2, 6, 16384, "fp32")])
def test_wide_rows_and_many_rows(oracle_mod, W, M, H, dtype):
    """The fused consumer with 4 and 8 vectors per thread: rows up to 8192 vectors for W <= 4
    and 4096 beyond, and the few-partial shapes the planner gives when rows outnumber CUs.  Round
    2 (the last buffer, the largest offsets; its push empties buffer 0)."""
    print("case", W, M, H, dtype, flush=True)
    parts, res, gam = synth.custom(W, M, H, dtype, seed=W + M + H)
    tdt = synth.TORCH_DTYPES[dtype]
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    rbuf = _new_rbuf(W, M, H, tdt)
    d_parts = [dev(p) for p in parts]
    for r, p in enumerate(d_parts):
        ar.ar_lamport_push(p, r, rbuf, 2)
    d_res = dev(res)
    ro, no = torch.empty_like(d_res), torch.empty_like(d_res)
    ar.ar_lamport_residual_rmsnorm(rbuf, 2, d_res, dev(gam), 1e-6, ro, no, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    check_round_state(rbuf, 2, d_parts)
    assert _empty(rbuf[1])
    want_ro, want_no = oracle_mod.ar_residual_rmsnorm([host_np(p) for p in parts], host_np(res),
                                                      gam.numpy(), 1e-6, dtype)
    assert_bit_exact(host_np(ro.cpu()), want_ro, dtype, "lamport residual_out")
    assert_norm_close(host_np(no.cpu()), want_no, dtype, "lamport norm_out")


FEW_ROWS = [(8, 1, 7168, "bf16"), (2, 64, 7168, "bf16"), (16, 48, 7168, "bf16"),
            (64, 16, 7168, "bf16"), (32, 64, 8192, "fp16"), (8, 32, 7168, "fp32"),
            (4, 7, 7176, "bf16"), (8, 3, 16376, "fp16")]


@pytest.mark.parametrize("W,M,H,dtype", FEW_ROWS, ids=["W%d-M%d-H%d-%s" % c for c in FEW_ROWS])
def test_few_rows_fewest_vectors_per_thread(oracle_mod, W, M, H, dtype):
    """Few rows (a quarter of the CUs or fewer): the fused consumer runs one or two vectors per
    thread over up to 1024 lanes, ragged widths (897 and 2047 vectors) included; four rounds, so
    the rotation wraps."""
    print("case", W, M, H, dtype, flush=True)
    tdt = synth.TORCH_DTYPES[dtype]
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    rbuf = _new_rbuf(W, M, H, tdt)
    for rnd in range(4):
        parts, res, gam = synth.custom(W, M, H, dtype, seed=W * 31 + M + H + rnd)
        d_parts = [dev(p) for p in parts]
        for r, p in enumerate(d_parts):
            ar.ar_lamport_push(p, r, rbuf, rnd)
        d_res = dev(res)
        ro, no = torch.empty_like(d_res), torch.empty_like(d_res)
        ar.ar_lamport_residual_rmsnorm(rbuf, rnd, d_res, dev(gam), 1e-6, ro, no, status)
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        check_round_state(rbuf, rnd, d_parts)
        want_ro, want_no = oracle_mod.ar_residual_rmsnorm(
            [host_np(p) for p in parts], host_np(res), gam.numpy(), 1e-6, dtype)
        assert_bit_exact(host_np(ro.cpu()), want_ro, dtype, "lamport residual_out")
        assert_norm_close(host_np(no.cpu()), want_no, dtype, "lamport norm_out")


def test_largest_round_number(oracle_mod):
    """Round 2^63 - 1 (buffer 1; its push empties buffer 2): the buffer arithmetic does not
    overflow at the largest round the ABI takes."""
    W, M, H, dtype = 4, 3, 1024, "bf16"
    rnd = 2 ** 63 - 1
    parts, res, gam = synth.custom(W, M, H, dtype, seed=63)
    tdt = synth.TORCH_DTYPES[dtype]
    d_parts = [dev(p) for p in parts]
    rbuf = _new_rbuf(W, M, H, tdt)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    for r, p in enumerate(d_parts):
        ar.ar_lamport_push(p, r, rbuf, rnd)
    d_res = dev(res)
    ro, no = torch.empty_like(d_res), torch.empty_like(d_res)
    ar.ar_lamport_residual_rmsnorm(rbuf, rnd, d_res, dev(gam), 1e-6, ro, no, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert rnd % NBUF == 1
    check_round_state(rbuf, rnd, d_parts)
    assert _empty(rbuf[0])
    want_ro, want_no = oracle_mod.ar_residual_rmsnorm([host_np(p) for p in parts], host_np(res),
                                                      gam.numpy(), 1e-6, dtype)
    assert_bit_exact(host_np(ro.cpu()), want_ro, dtype, "residual_out")
    assert_norm_close(host_np(no.cpu()), want_no, dtype, "norm_out")
