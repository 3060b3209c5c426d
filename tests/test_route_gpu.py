"""The routed entry point on the GPU: calls whose route is one-shot, two-shot (every rank's share,
then the all-gather), the two-kernel path and the fallback, each against the oracle (out and
residual_out bit-identical, norm_out within 1 ulp) or, for the fallback, the error and untouched
outputs.
"""
import pytest
import torch

import all_reduce_residual_amd as ar
import synth
from gpu_util import assert_bit_exact, assert_norm_close, dev, host_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    ar.lib()


def _case(W, M, H, dtype, seed):
    parts, res, gam = synth.custom(W, M, H, dtype, seed=seed)
    return parts, res, gam, [dev(p) for p in parts], dev(res), dev(gam)


def _want(oracle_mod, pattern, parts, res, gam, eps, dtype):
    hp = [host_np(p) for p in parts]
    if pattern == "sum":
        return (oracle_mod.ar_sum(hp, dtype),)
    return oracle_mod.ar_residual_rmsnorm(hp, host_np(res), gam.numpy(), eps, dtype)


def _check(got, want, pattern, dtype, what):
    assert_bit_exact(host_np(got[0].cpu()), want[0], dtype, what + " out/residual_out")
    if pattern == "rms":
        assert_norm_close(host_np(got[1].cpu()), want[1], dtype, what + " norm_out")


def _routed(pattern, d_parts, d_res, d_gam, eps, outs, rank=0, policy=None):
    if pattern == "sum":
        return ar.ar_allreduce_routed(d_parts, outs[0], rank=rank, policy=policy)
    return ar.ar_allreduce_routed(d_parts, outs[0], residual=d_res, gamma=d_gam, eps=eps,
                                  norm_out=outs[1], rank=rank, policy=policy)


def _outs(pattern, like):
    return [torch.full_like(like, 3.0) for _ in range(1 if pattern == "sum" else 2)]


@pytest.mark.parametrize("pattern", ["sum", "rms"])
@pytest.mark.parametrize("W,M,H,dtype", [(8, 16, 7168, "bf16"), (2, 4, 256, "bf16"),
                                         (16, 8, 8192, "fp16"), (4, 5, 1024, "fp32")])
def test_one_shot_route(oracle_mod, pattern, W, M, H, dtype):
    print("case one-shot", pattern, W, M, H, dtype, flush=True)
    parts, res, gam, dp, dr, dg = _case(W, M, H, dtype, seed=W * 7 + M)
    outs = _outs(pattern, dr)
    assert _routed(pattern, dp, dr, dg, 1e-6, outs) == ar.ROUTE_ONE_SHOT
    torch.cuda.synchronize()
    _check(outs, _want(oracle_mod, pattern, parts, res, gam, 1e-6, dtype), pattern, dtype,
           "one-shot")


@pytest.mark.parametrize("pattern", ["sum", "rms"])
@pytest.mark.parametrize("W,M,H,dtype", [(8, 2048, 7168, "bf16"), (4, 301, 4096, "fp16")])
def test_two_shot_route_shares_then_gather(oracle_mod, pattern, W, M, H, dtype):
    """Every rank's share writes its row slice in place; the gather (slices already in place, so
    skipped) completes the call.  One rank's share alone leaves every other row untouched."""
    print("case two-shot", pattern, W, M, H, dtype, flush=True)
    parts, res, gam, dp, dr, dg = _case(W, M, H, dtype, seed=W * 11 + M)
    policy = dict(ar.ar_policy_default(W), two_shot_min_bytes=0, min_tokens=1)
    # One share alone.
    outs = _outs(pattern, dr)
    assert _routed(pattern, dp, dr, dg, 1e-6, outs, rank=W - 1, policy=policy) == \
        ar.ROUTE_TWO_SHOT
    torch.cuda.synchronize()
    b, c = ar.ar_row_partition(W, M, W - 1)
    for o in outs:
        assert bool((o[:b].float() == 3.0).all()) and bool((o[b + c:].float() == 3.0).all())
    want = _want(oracle_mod, pattern, parts, res, gam, 1e-6, dtype)
    assert_bit_exact(host_np(outs[0][b:b + c].cpu()), want[0][b:b + c], dtype, "share rows")
    # All shares, then the gather.
    outs = _outs(pattern, dr)
    for rank in range(W):
        assert _routed(pattern, dp, dr, dg, 1e-6, outs, rank=rank, policy=policy) == \
            ar.ROUTE_TWO_SHOT
    for o in outs:
        slices = []
        for j in range(W):
            bj, cj = ar.ar_row_partition(W, M, j)
            slices.append(o[bj:bj + cj])
        ar.ar_all_gather(slices, o)
    torch.cuda.synchronize()
    _check(outs, want, pattern, dtype, "two-shot")


def test_default_policy_routes_the_wide_hidden_call_to_two_shot():
    W, M, H = 8, 2048, 7168
    assert ar.ar_route(ar.PATTERN_AR_RESIDUAL_RMSNORM, W, M, H, ar.DTYPE_BF16) == \
        ar.ROUTE_TWO_SHOT


@pytest.mark.parametrize("W,M,H,dtype", [(8, 33, 7170, "bf16"), (2, 7, 65544, "bf16"),
                                         (4, 9, 1023, "fp32")])
def test_unfused_route(oracle_mod, W, M, H, dtype):
    """Norm rows the fused kernel does not take (odd width, above the fused limit) run the
    two-kernel path."""
    print("case unfused", W, M, H, dtype, flush=True)
    parts, res, gam, dp, dr, dg = _case(W, M, H, dtype, seed=W + M + H)
    outs = _outs("rms", dr)
    assert _routed("rms", dp, dr, dg, 1e-5, outs) == ar.ROUTE_UNFUSED
    torch.cuda.synchronize()
    _check(outs, _want(oracle_mod, "rms", parts, res, gam, 1e-5, dtype), "rms", dtype,
           "unfused")


@pytest.mark.parametrize("pattern", ["sum", "rms"])
def test_fallback_route_launches_nothing(pattern):
    """World size 12 is not taken here: AR_ERR_UNSUPPORTED and the outputs stay as they were."""
    W, M, H, dtype = 12, 4, 1024, "bf16"
    _, _, _, dp, dr, dg = _case(W, M, H, dtype, seed=12)
    outs = _outs(pattern, dr)
    with pytest.raises(ar.ArError) as e:
        _routed(pattern, dp, dr, dg, 1e-6, outs)
    assert e.value.status == ar.AR_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    for o in outs:
        assert bool((o.float() == 3.0).all())
