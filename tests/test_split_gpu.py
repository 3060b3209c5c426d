"""Parity of the split-row kARResidualRMSNorm kernel (several blocks per row, partial sums of
squares exchanged through a caller workspace) with the oracle, through the C ABI.

Bar as for the one-block-per-row kernel: residual_out bit-identical, norm_out within 1 ulp
(16-bit) or 1e-5 relative (binary32).  Also checked: a block that stops waiting (max_polls = 0
forces it from the host) gives bit-identical results; one workspace serves calls of changing
shape, graph replays and a cleared workspace; the planned entry point runs in-place calls on the
one-block-per-row kernel; the workspace's tags advance as documented.
"""
import numpy as np
import pytest
import torch

import all_reduce_residual_amd as ar
import synth
from gpu_util import assert_bit_exact, assert_norm_close, dev, host_np

pytestmark = pytest.mark.gpu

TD = synth.TORCH_DTYPES
VEC = {"bf16": 8, "fp16": 8, "fp32": 4}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    ar.lib()


def _cfg(H, dtype, threads, vpt, polls=1 << 14):
    V = H // VEC[dtype]
    return {"threads_per_block": threads, "vecs_per_thread": vpt,
            "segments": -(-V // (threads * vpt)), "max_polls": polls}


def _run(parts, res, gam, eps, ws, config=None):
    d_parts = [dev(p) for p in parts]
    d_res, d_gam = dev(res), dev(gam)
    ro, no = torch.empty_like(d_res), torch.empty_like(d_res)
    ar.ar_residual_rmsnorm_ws(d_parts, d_res, d_gam, eps, ro, no, ws, config=config)
    torch.cuda.synchronize()
    return host_np(ro.cpu()), host_np(no.cpu())


def _check(oracle_mod, parts, res, gam, eps, dtype, ro, no):
    want_ro, want_no = oracle_mod.ar_residual_rmsnorm([host_np(p) for p in parts], host_np(res),
                                                      gam.numpy(), eps, dtype)
    assert_bit_exact(ro, want_ro, dtype, "residual_out")
    assert_norm_close(no, want_no, dtype)


# (W, M, H, threads, vpt): single-wave segments, two-vector segments, multi-wave segments, a
# ragged last segment (H = 1032: 129 vectors), one segment per row, 64 segments per row.
CASES = [
    (8, 1, 7168, 64, 1), (8, 5, 7168, 64, 2), (8, 3, 7168, 128, 1), (8, 2, 7168, 256, 2),
    (4, 7, 1032, 64, 1), (2, 4, 4096, 64, 1), (1, 3, 4096, 128, 2), (16, 2, 8192, 64, 2),
    (32, 2, 2048, 64, 1), (64, 1, 1024, 64, 1), (8, 2, 512, 1024, 1), (2, 1, 32768, 512, 1),
]


@pytest.mark.parametrize("W,M,H,threads,vpt", CASES,
                         ids=["W%d-M%d-H%d-L%d-v%d" % c for c in CASES])
@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_split_matches_oracle(oracle_mod, W, M, H, threads, vpt, dtype):
    if dtype == "fp32" and H // 4 > threads * vpt * ar.SPLIT_SLOTS:
        pytest.skip("more than 64 segments")
    print("case split", W, M, H, threads, vpt, dtype, flush=True)
    parts, res, gam = synth.custom(W, M, H, dtype, seed=31 * H + 7 * M + W)
    ws = ar.new_workspace(M, "cuda")
    ro, no = _run(parts, res, gam, 1e-6, ws, _cfg(H, dtype, threads, vpt))
    _check(oracle_mod, parts, res, gam, 1e-6, dtype, ro, no)


@pytest.mark.parametrize("M", [7, 8, 9, 1000, 65535])
def test_split_grid_forms_and_row_limit(oracle_mod, M):
    """Both grid forms (8 x S blocks below 8 rows, one row's segments on one XCD; S x M from 8
    rows) and the most rows the S x M grid takes (65535, its y limit), two segments per row,
    every row against the oracle."""
    W, H, dtype = 2, 1024, "bf16"
    print("case split grid W=%d M=%d H=%d" % (W, M, H), flush=True)
    parts, res, gam = synth.custom(W, M, H, dtype, seed=M)
    cfg = _cfg(H, dtype, 64, 1)
    assert cfg["segments"] == 2
    ro, no = _run(parts, res, gam, 1e-6, ar.new_workspace(M, "cuda"), config=cfg)
    _check(oracle_mod, parts, res, gam, 1e-6, dtype, ro, no)


@pytest.mark.parametrize("M", [1, 8, 32, 64, 128])
def test_wide_hidden_decode_sizes_planned(oracle_mod, M):
    """The wide-hidden workload (W = 8, H = 7168 bf16) at decode sizes, planned shape."""
    print("case split wide_hidden", M, flush=True)
    wl = synth.WORKLOADS["wide_hidden"]
    parts, res, gam = synth.inputs(wl, M)
    ws = ar.new_workspace(M, "cuda")
    ro, no = _run(parts, res, gam, wl.eps, ws)
    _check(oracle_mod, parts, res, gam, wl.eps, "bf16", ro, no)


PLANNED = [(16, 4, 8192, "fp16"), (4, 32, 8192, "bf16"), (64, 2, 4096, "bf16"),
           (32, 3, 8192, "fp32"), (16, 100, 8192, "bf16"), (8, 64, 7168, "fp16"),
           (8, 80, 7168, "bf16"), (8, 112, 8192, "fp16")]


@pytest.mark.parametrize("W,M,H,dtype", PLANNED, ids=["W%d-M%d-H%d-%s" % c for c in PLANNED])
def test_planned_splits_match_oracle(oracle_mod, W, M, H, dtype):
    """Shapes the heuristic splits (2 to 16 segments), through the planned entry point."""
    cfg = ar.ar_split_config(W, M, H, {"bf16": ar.DTYPE_BF16, "fp16": ar.DTYPE_FP16,
                                       "fp32": ar.DTYPE_FP32}[dtype])
    assert cfg["segments"] >= 2, cfg
    print("case split planned", W, M, H, dtype, cfg, flush=True)
    parts, res, gam = synth.custom(W, M, H, dtype, seed=13 * W + M)
    ws = ar.new_workspace(M, "cuda")
    ro, no = _run(parts, res, gam, 1e-6, ws)
    _check(oracle_mod, parts, res, gam, 1e-6, dtype, ro, no)
    assert (_tags(ws, M) == 1).all()


def test_fp16_outliers_many_ranks(oracle_mod):
    print("case split fp16 outliers", flush=True)
    wl = synth.WORKLOADS["fp16_many_rank"]
    parts, res, gam = synth.inputs(wl, 4)
    ws = ar.new_workspace(4, "cuda")
    ro, no = _run(parts, res, gam, wl.eps, ws, _cfg(wl.H, "fp16", 64, 1))
    _check(oracle_mod, parts, res, gam, wl.eps, "fp16", ro, no)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("threads,vpt", [(64, 1), (128, 2)])
def test_blocks_that_stop_waiting_give_identical_results(threads, vpt, dtype):
    """max_polls = 0: no block waits, each reads the whole row and sums every segment's squares
    itself in the exchange's order; outputs must be bit-identical to the exchanged run."""
    print("case split no-wait", threads, vpt, dtype, flush=True)
    parts, res, gam = synth.custom(8, 6, 7168, dtype, seed=99)
    ws = ar.new_workspace(6, "cuda")
    ro_a, no_a = _run(parts, res, gam, 1e-6, ws, _cfg(7168, dtype, threads, vpt))
    ro_b, no_b = _run(parts, res, gam, 1e-6, ws, _cfg(7168, dtype, threads, vpt, polls=0))
    assert_bit_exact(ro_b, ro_a, dtype, "residual_out")
    assert_bit_exact(no_b, no_a, dtype, "norm_out")


def _tags(ws, M):
    w = ws.view(torch.int64).cpu().numpy().view(np.uint64).reshape(-1, ar.SPLIT_SLOTS)[:M]
    return (w >> np.uint64(32)).astype(np.int64)


def test_one_workspace_across_shapes_and_calls(oracle_mod):
    """Changing segment counts and row counts on one workspace: every call correct, and after
    each call every slot of each row it used carries that row's call count."""
    ws = ar.new_workspace(16, "cuda")
    uses = np.zeros(16, dtype=np.int64)
    seq = [(16, 64, 1), (4, 256, 2), (16, 64, 1), (9, 128, 1), (1, 1024, 1), (16, 64, 2),
           (3, 64, 1)]
    for i, (M, threads, vpt) in enumerate(seq):
        print("case split sequence", i, M, threads, vpt, flush=True)
        parts, res, gam = synth.custom(8, M, 7168, "bf16", seed=500 + i)
        ro, no = _run(parts, res, gam, 1e-6, ws, _cfg(7168, "bf16", threads, vpt))
        _check(oracle_mod, parts, res, gam, 1e-6, "bf16", ro, no)
        uses[:M] += 1
        tags = _tags(ws, 16)
        assert (tags == uses[:, None]).all(), (i, tags[:, 0], uses)


def test_cleared_workspace_after_garbage(oracle_mod):
    """A workspace full of stale data, cleared with ar_workspace_clear, serves correctly."""
    print("case split clear", flush=True)
    ws = torch.randint(0, 255, (ar.split_workspace_bytes(8),), dtype=torch.uint8, device="cuda")
    ar.ar_workspace_clear(ws)
    torch.cuda.synchronize()
    assert int(ws.count_nonzero()) == 0
    parts, res, gam = synth.custom(4, 8, 4096, "bf16", seed=77)
    ro, no = _run(parts, res, gam, 1e-6, ws, _cfg(4096, "bf16", 64, 1))
    _check(oracle_mod, parts, res, gam, 1e-6, "bf16", ro, no)


def test_graph_replays():
    """A captured split call replayed several times with eager work between replays: the tags
    advance on the device and every replay equals the eager result."""
    print("case split graph", flush=True)
    M, H = 4, 7168
    parts, res, gam = synth.custom(8, M, H, "bf16", seed=1234)
    d_parts = [dev(p) for p in parts]
    d_res, d_gam = dev(res), dev(gam)
    ws = ar.new_workspace(M, "cuda")
    ro0, no0 = torch.empty_like(d_res), torch.empty_like(d_res)
    ar.ar_residual_rmsnorm_ws(d_parts, d_res, d_gam, 1e-6, ro0, no0, ws)
    torch.cuda.synchronize()
    ro, no = torch.empty_like(d_res), torch.empty_like(d_res)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ar.ar_residual_rmsnorm_ws(d_parts, d_res, d_gam, 1e-6, ro, no, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ar.ar_residual_rmsnorm_ws(d_parts, d_res, d_gam, 1e-6, ro, no, ws)
    for i in range(4):
        ro.fill_(0)
        no.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ro.view(torch.int16), ro0.view(torch.int16)), i
        assert torch.equal(no.view(torch.int16), no0.view(torch.int16)), i
    assert (_tags(ws, M) == 2 + 4).all()


def test_in_place_runs_one_block_per_row(oracle_mod):
    """residual_out == residual: the planned entry point keeps one block per row (a block that
    stopped waiting would re-read overwritten residual values); the explicit split refuses."""
    print("case split in-place", flush=True)
    M, H = 4, 7168
    parts, res, gam = synth.custom(8, M, H, "bf16", seed=4321)
    d_parts = [dev(p) for p in parts]
    d_res, d_gam = dev(res), dev(gam)
    no = torch.empty_like(d_res)
    ws = ar.new_workspace(M, "cuda")
    with pytest.raises(ar.ArError) as e:
        ar.ar_residual_rmsnorm_ws(d_parts, d_res, d_gam, 1e-6, d_res, no, ws,
                                  config=_cfg(H, "bf16", 64, 1))
    assert e.value.status == ar.AR_ERR_ALIAS
    ar.ar_residual_rmsnorm_ws(d_parts, d_res, d_gam, 1e-6, d_res, no, ws)
    torch.cuda.synchronize()
    _check(oracle_mod, parts, res, gam, 1e-6, "bf16", host_np(d_res.cpu()), host_np(no.cpu()))
    assert (_tags(ws, M) == 0).all()


def test_planned_large_m_matches_fused_kernel():
    """Where the planner keeps one block per row, the workspace entry point is the plain fused
    call: bit-identical outputs."""
    print("case split planned large M", flush=True)
    M, H = 1024, 7168
    assert ar.ar_split_config(8, M, H, ar.DTYPE_BF16)["segments"] == 0
    parts, res, gam = synth.custom(8, M, H, "bf16", seed=2024)
    d_parts = [dev(p) for p in parts]
    d_res, d_gam = dev(res), dev(gam)
    ws = ar.new_workspace(M, "cuda")
    ro_a, no_a = torch.empty_like(d_res), torch.empty_like(d_res)
    ro_b, no_b = torch.empty_like(d_res), torch.empty_like(d_res)
    ar.ar_residual_rmsnorm_ws(d_parts, d_res, d_gam, 1e-6, ro_a, no_a, ws)
    ar.ar_residual_rmsnorm(d_parts, d_res, d_gam, 1e-6, ro_b, no_b)
    torch.cuda.synchronize()
    assert torch.equal(ro_a.view(torch.int16), ro_b.view(torch.int16))
    assert torch.equal(no_a.view(torch.int16), no_b.view(torch.int16))
