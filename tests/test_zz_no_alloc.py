"""The no-allocation entry point against the workspace form it shares its kernels with.

ar_residual_rmsnorm_noalloc keeps the split kernel's exchange slots in a device array of the
library instead of a caller workspace.  Two calls in a row -- the second with fewer rows, so the
array holds the first call's state -- must each give what ar_residual_rmsnorm_ws gives with a
fresh caller workspace (residual_out and norm_out bit-identical: the same kernel and launch
shape), and what the oracle gives (residual_out bit-identical, norm_out within the norm bar).
"""
import pytest
import torch

import all_reduce_residual_amd as ar
import synth
from gpu_util import assert_bit_exact, assert_norm_close, dev, host_np

pytestmark = pytest.mark.gpu

# (W, M, H, element type): the planner splits these rows over several blocks, then fewer rows.
CALLS = [(8, 16, 7168, "bf16"), (8, 3, 7168, "bf16"), (16, 9, 8192, "fp16"), (8, 1, 7168, "fp32")]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    ar.lib()


def test_noalloc_matches_workspace_form(oracle_mod):
    for i, (W, M, H, dtype) in enumerate(CALLS):
        print("case noalloc call", i, W, M, H, dtype, flush=True)
        code = {"bf16": ar.DTYPE_BF16, "fp16": ar.DTYPE_FP16, "fp32": ar.DTYPE_FP32}[dtype]
        assert ar.ar_split_config(W, M, H, code)["segments"] > 1
        parts, res, gam = synth.custom(W, M, H, dtype, seed=31 + i)
        d_parts, d_res, d_gam = [dev(p) for p in parts], dev(res), dev(gam)
        ro_a, no_a = torch.empty_like(d_res), torch.empty_like(d_res)
        ro_b, no_b = torch.empty_like(d_res), torch.empty_like(d_res)
        ws = ar.new_workspace(M, "cuda")
        torch.cuda.synchronize()
        ar.ar_residual_rmsnorm_ws(d_parts, d_res, d_gam, 1e-6, ro_a, no_a, ws)
        ar.ar_residual_rmsnorm_noalloc(d_parts, d_res, d_gam, 1e-6, ro_b, no_b)
        torch.cuda.synchronize()
        assert_bit_exact(host_np(ro_b.cpu()), host_np(ro_a.cpu()), dtype, "residual_out")
        assert_bit_exact(host_np(no_b.cpu()), host_np(no_a.cpu()), dtype, "norm_out")
        want_ro, want_no = oracle_mod.ar_residual_rmsnorm([host_np(p) for p in parts],
                                                          host_np(res), gam.numpy(), 1e-6, dtype)
        assert_bit_exact(host_np(ro_b.cpu()), want_ro, dtype, "residual_out vs oracle")
        assert_norm_close(host_np(no_b.cpu()), want_no, dtype)


def test_noalloc_most_rows_accepted(oracle_mod):
    """The largest row count the array is sized for runs and matches the oracle."""
    W, M, H, dtype = 2, ar.NOALLOC_MAX_ROWS, 256, "bf16"
    print("case noalloc rows", M, flush=True)
    parts, res, gam = synth.custom(W, M, H, dtype, seed=6)
    d_parts, d_res = [dev(p) for p in parts], dev(res)
    ro, no = torch.empty_like(d_res), torch.empty_like(d_res)
    ar.ar_residual_rmsnorm_noalloc(d_parts, d_res, dev(gam), 1e-6, ro, no)
    torch.cuda.synchronize()
    want_ro, want_no = oracle_mod.ar_residual_rmsnorm([host_np(p) for p in parts], host_np(res),
                                                      gam.numpy(), 1e-6, dtype)
    assert_bit_exact(host_np(ro.cpu()), want_ro, dtype, "residual_out")
    assert_norm_close(host_np(no.cpu()), want_no, dtype)


def test_noalloc_rows_beyond_the_array_rejected():
    W, M, H = 2, ar.NOALLOC_MAX_ROWS + 1, 256
    parts, res, gam = synth.custom(W, M, H, "bf16", seed=5)
    d_parts, d_res = [dev(p) for p in parts], dev(res)
    ro, no = torch.empty_like(d_res), torch.empty_like(d_res)
    with pytest.raises(ar.ArError) as e:
        ar.ar_residual_rmsnorm_noalloc(d_parts, d_res, dev(gam), 1e-6, ro, no)
    assert e.value.status == ar.AR_ERR_UNSUPPORTED


def test_noalloc_replayed_from_a_graph(oracle_mod):
    """Captured once (after an eager call, the usual warm-up before capture) and replayed with
    new inputs, with eager no-alloc calls of another shape between the replays: the array keeps
    whatever the last call left and every replay still matches the oracle."""
    W, M, H, dtype = 8, 16, 7168, "bf16"
    parts, res, gam = synth.custom(W, M, H, dtype, seed=71)
    d_parts, d_res, d_gam = [dev(p) for p in parts], dev(res), dev(gam)
    ro, no = torch.empty_like(d_res), torch.empty_like(d_res)
    o_parts, o_res, o_gam = synth.custom(W, 5, H, dtype, seed=72)
    do_parts, do_res, do_gam = [dev(p) for p in o_parts], dev(o_res), dev(o_gam)
    o_ro, o_no = torch.empty_like(do_res), torch.empty_like(do_res)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ar.ar_residual_rmsnorm_noalloc(d_parts, d_res, d_gam, 1e-6, ro, no)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ar.ar_residual_rmsnorm_noalloc(d_parts, d_res, d_gam, 1e-6, ro, no)
    for rep in range(3):
        print("case noalloc graph replay", rep, flush=True)
        p2, r2, _ = synth.custom(W, M, H, dtype, seed=80 + rep)
        for d, h in zip(d_parts + [d_res], p2 + [r2]):
            d.copy_(h)
        ar.ar_residual_rmsnorm_noalloc(do_parts, do_res, do_gam, 1e-6, o_ro, o_no)
        graph.replay()
        torch.cuda.synchronize()
        want_ro, want_no = oracle_mod.ar_residual_rmsnorm([host_np(p) for p in p2], host_np(r2),
                                                          gam.numpy(), 1e-6, dtype)
        assert_bit_exact(host_np(ro.cpu()), want_ro, dtype, "replay %d residual_out" % rep)
        assert_norm_close(host_np(no.cpu()), want_no, dtype, "replay %d norm_out" % rep)
        want_ro, want_no = oracle_mod.ar_residual_rmsnorm([host_np(p) for p in o_parts],
                                                          host_np(o_res), o_gam.numpy(), 1e-6,
                                                          dtype)
        assert_bit_exact(host_np(o_ro.cpu()), want_ro, dtype, "eager call %d residual_out" % rep)
        assert_norm_close(host_np(o_no.cpu()), want_no, dtype, "eager call %d norm_out" % rep)
