"""Lamport-style one-shot exchange on the GPU: producers push their partials into the slots of
a receive buffer, the consumer polls, reduces exactly like the plain entry points and empties
the slots again.  Results are compared with the oracle (bit-identical out/residual_out, norm_out
within 1 ulp); every wait is bounded, and the one test that exercises a timeout forces it from
the host with a spin limit of 4 polls (the kernel still finishes).
"""
import numpy as np
import pytest
import torch

import all_reduce_residual_amd as ar
import synth
from gpu_util import assert_bit_exact, assert_norm_close, dev, host_np

pytestmark = pytest.mark.gpu

ALL_ONES = {torch.bfloat16: -1, torch.float16: -1, torch.float32: -1}   # int view of all ones


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    ar.lib()


def _int_view(t):
    return t.view(torch.int32 if t.dtype == torch.float32 else torch.int16)


def _empty(rbuf):
    return bool((_int_view(rbuf) == -1).all())


def _new_rbuf(W, M, H, tdt):
    rbuf = torch.empty((W, M, H), dtype=tdt, device="cuda")
    ar.ar_lamport_arm(rbuf)
    return rbuf


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
        ar.ar_lamport_push(p, r, rbuf)
    out = torch.empty_like(d_parts[0])
    ar.ar_lamport_sum(rbuf, out, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0 and _empty(rbuf)
    assert_bit_exact(host_np(out.cpu()), oracle_mod.ar_sum(hp, dtype), dtype, "lamport out")
    for r, p in enumerate(d_parts):
        ar.ar_lamport_push(p, r, rbuf)
    d_res, d_gam = dev(res), dev(gam)
    ro, no = torch.empty_like(d_res), torch.empty_like(d_res)
    ar.ar_lamport_residual_rmsnorm(rbuf, d_res, d_gam, 1e-6, ro, no, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0 and _empty(rbuf)
    want_ro, want_no = oracle_mod.ar_residual_rmsnorm(hp, host_np(res), gam.numpy(), 1e-6, dtype)
    assert_bit_exact(host_np(ro.cpu()), want_ro, dtype, "lamport residual_out")
    assert_norm_close(host_np(no.cpu()), want_no, dtype, "lamport norm_out")


def test_rounds_reuse_the_buffer(oracle_mod):
    """The consumer leaves the buffer empty, so rounds follow each other without re-arming."""
    W, M, H, dtype = 8, 33, 7168, "bf16"
    tdt = synth.TORCH_DTYPES[dtype]
    rbuf = _new_rbuf(W, M, H, tdt)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    for rnd in range(3):
        parts, res, gam = synth.custom(W, M, H, dtype, seed=50 + rnd)
        d_parts = [dev(p) for p in parts]
        for r, p in enumerate(d_parts):
            ar.ar_lamport_push(p, r, rbuf)
        d_res, d_gam = dev(res), dev(gam)
        ro, no = torch.empty_like(d_res), torch.empty_like(d_res)
        ar.ar_lamport_residual_rmsnorm(rbuf, d_res, d_gam, 1e-6, ro, no, status)
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        want_ro, want_no = oracle_mod.ar_residual_rmsnorm([host_np(p) for p in parts],
                                                          host_np(res), gam.numpy(), 1e-6, dtype)
        assert_bit_exact(host_np(ro.cpu()), want_ro, dtype, "round %d residual_out" % rnd)
        assert_norm_close(host_np(no.cpu()), want_no, dtype, "round %d norm_out" % rnd)
    assert _empty(rbuf)


@pytest.mark.parametrize("pattern", ["sum", "rms"])
def test_consumer_polls_while_producers_run(oracle_mod, pattern):
    """Producers on one stream, delayed by a sleep kernel, and the consumer on another.  Streams
    share the GPU's few hardware queues, so only this order is safe whatever the mapping: on
    separate queues the consumer starts first and polls until the pushes land; on one queue the
    pushes simply run first."""
    W, M, H, dtype = 8, 8, 7168, "bf16"
    tdt = synth.TORCH_DTYPES[dtype]
    parts, res, gam = synth.custom(W, M, H, dtype, seed=77)
    d_parts = [dev(p) for p in parts]
    d_res, d_gam = dev(res), dev(gam)
    rbuf = _new_rbuf(W, M, H, tdt)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    out, ro, no = (torch.empty_like(d_res) for _ in range(3))
    consumer, producer = torch.cuda.Stream(), torch.cuda.Stream()
    for st in (consumer, producer):       # first use of a stream can take milliseconds
        with torch.cuda.stream(st):
            torch.zeros(1, device="cuda").add_(1)
    torch.cuda.synchronize()
    with torch.cuda.stream(producer):
        torch.cuda._sleep(1 << 20)            # ~0.5 ms on the producer stream
    for r, p in enumerate(d_parts):
        ar.ar_lamport_push(p, r, rbuf, stream=producer)
    if pattern == "sum":
        ar.ar_lamport_sum(rbuf, out, status, spin_limit=1 << 20, stream=consumer)
    else:
        ar.ar_lamport_residual_rmsnorm(rbuf, d_res, d_gam, 1e-6, ro, no, status,
                                       spin_limit=1 << 20, stream=consumer)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    hp = [host_np(p) for p in parts]
    if pattern == "sum":
        assert_bit_exact(host_np(out.cpu()), oracle_mod.ar_sum(hp, dtype), dtype, "out")
    else:
        want_ro, want_no = oracle_mod.ar_residual_rmsnorm(hp, host_np(res), gam.numpy(), 1e-6,
                                                          dtype)
        assert_bit_exact(host_np(ro.cpu()), want_ro, dtype, "residual_out")
        assert_norm_close(host_np(no.cpu()), want_no, dtype)
    assert _empty(rbuf)


def test_missing_producer_times_out_and_reports():
    """One rank never pushes: with a spin limit of 4 polls the consumer gives up, sets the status
    bit and finishes (forced from the host; no unbounded wait exists)."""
    W, M, H = 4, 2, 256
    parts, _, _ = synth.custom(W, M, H, "bf16", seed=5, with_norm=False)
    rbuf = _new_rbuf(W, M, H, torch.bfloat16)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    for r, p in enumerate(parts[:-1]):
        ar.ar_lamport_push(dev(p), r, rbuf)
    out = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
    ar.ar_lamport_sum(rbuf, out, status, spin_limit=4)
    torch.cuda.synchronize()
    assert int(status.item()) & 1 == 1
    ar.ar_lamport_arm(rbuf)
    torch.cuda.synchronize()
    assert _empty(rbuf)


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
        ar.ar_lamport_push(p, r, rbuf)
    out = torch.empty_like(d_parts[0])
    ar.ar_lamport_sum(rbuf, out, status, spin_limit=64)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
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
    for r, p in enumerate(parts):
        ar.ar_lamport_push(dev(p), r, rbuf)
    d_res, d_gam = dev(res), dev(gam)
    ro, no = torch.empty_like(d_res), torch.empty_like(d_res)
    ar.ar_lamport_residual_rmsnorm(rbuf, d_res, d_gam, wl.eps, ro, no, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0 and _empty(rbuf)
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
    and 4096 beyond, and the few-partial shapes the planner gives when rows outnumber CUs."""
    print("case", W, M, H, dtype, flush=True)
    parts, res, gam = synth.custom(W, M, H, dtype, seed=W + M + H)
    tdt = synth.TORCH_DTYPES[dtype]
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    rbuf = _new_rbuf(W, M, H, tdt)
    for r, p in enumerate(parts):
        ar.ar_lamport_push(dev(p), r, rbuf)
    d_res = dev(res)
    ro, no = torch.empty_like(d_res), torch.empty_like(d_res)
    ar.ar_lamport_residual_rmsnorm(rbuf, d_res, dev(gam), 1e-6, ro, no, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0 and _empty(rbuf)
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
    thread over up to 1024 lanes, ragged widths (897 and 2047 vectors) included; then a second
    round through the re-armed buffer."""
    print("case", W, M, H, dtype, flush=True)
    tdt = synth.TORCH_DTYPES[dtype]
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    rbuf = _new_rbuf(W, M, H, tdt)
    for rnd in range(2):
        parts, res, gam = synth.custom(W, M, H, dtype, seed=W * 31 + M + H + rnd)
        for r, p in enumerate(parts):
            ar.ar_lamport_push(dev(p), r, rbuf)
        d_res = dev(res)
        ro, no = torch.empty_like(d_res), torch.empty_like(d_res)
        ar.ar_lamport_residual_rmsnorm(rbuf, d_res, dev(gam), 1e-6, ro, no, status)
        torch.cuda.synchronize()
        assert int(status.item()) == 0 and _empty(rbuf)
        want_ro, want_no = oracle_mod.ar_residual_rmsnorm(
            [host_np(p) for p in parts], host_np(res), gam.numpy(), 1e-6, dtype)
        assert_bit_exact(host_np(ro.cpu()), want_ro, dtype, "lamport residual_out")
        assert_norm_close(host_np(no.cpu()), want_no, dtype, "lamport norm_out")
