"""Two-shot share on the GPU: every rank's reduce-scatter share (the fused kernels on its row
slice) followed by the all-gather share reproduces the oracle's full result (residual_out and
out bit-identical, norm_out within 1 ulp); the gather itself is a bit-exact copy.
"""
import numpy as np
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


def two_shot(pattern, d_parts, d_res, d_gam, eps, in_place=False):
    """Run every rank's share on one GPU: reduce-scatter on row slices, then all-gather."""
    W = len(d_parts)
    M, H = d_parts[0].shape
    outs = {"out": torch.empty_like(d_parts[0])} if pattern == "sum" else \
        {"ro": torch.empty_like(d_res), "no": torch.empty_like(d_res)}
    slices = {k: [] for k in outs}
    for j in range(W):
        b, c = ar.ar_row_partition(W, M, j)
        sl = {}
        for k, full in outs.items():
            # In place: rank j writes straight into its rows of the gathered tensor.
            sl[k] = full[b:b + c] if in_place and j % 2 == 0 else \
                torch.empty((c, H), dtype=full.dtype, device="cuda")
            slices[k].append(sl[k])
        if c == 0:
            continue
        views = [p[b:b + c] for p in d_parts]
        if pattern == "sum":
            ar.ar_sum(views, sl["out"])
        else:
            ar.ar_residual_rmsnorm(views, d_res[b:b + c], d_gam, eps, sl["ro"], sl["no"])
    for k, full in outs.items():
        ar.ar_all_gather(slices[k], full)
    torch.cuda.synchronize()
    return outs


CASES = [("wide_hidden", 1), ("wide_hidden", 8), ("wide_hidden", 2048), ("llama3_decode", 128),
         ("large_sum", 5120), ("fp16_many_rank", 512), ("tiny", 4)]


@pytest.mark.parametrize("name,M", CASES, ids=["%s-M%d" % c for c in CASES])
def test_two_shot_matches_oracle(oracle_mod, name, M):
    wl = synth.WORKLOADS[name]
    print("case", name, M, flush=True)
    parts, res, gam = synth.inputs(wl, M)
    d_parts = [dev(p) for p in parts]
    hp = [host_np(p) for p in parts]
    for pattern in wl.patterns:
        if pattern == "sum":
            o = two_shot("sum", d_parts, None, None, None)
            assert_bit_exact(host_np(o["out"].cpu()), oracle_mod.ar_sum(hp, wl.dtype), wl.dtype,
                             "two-shot out")
        else:
            o = two_shot("rms", d_parts, dev(res), dev(gam), wl.eps, in_place=(M % 2 == 0))
            want_ro, want_no = oracle_mod.ar_residual_rmsnorm(hp, host_np(res), gam.numpy(),
                                                              wl.eps, wl.dtype)
            assert_bit_exact(host_np(o["ro"].cpu()), want_ro, wl.dtype, "two-shot residual_out")
            assert_norm_close(host_np(o["no"].cpu()), want_no, wl.dtype, "two-shot norm_out")


@pytest.mark.parametrize("W,M", [(8, 3), (16, 5), (64, 63), (4, 1), (2, 1)])
def test_fewer_rows_than_ranks(oracle_mod, W, M):
    """Empty slices (M < W) are skipped; the gathered result is still the full one."""
    parts, res, gam = synth.custom(W, M, 256, "bf16", seed=W * 100 + M)
    d_parts = [dev(p) for p in parts]
    o = two_shot("rms", d_parts, dev(res), dev(gam), 1e-6)
    want_ro, want_no = oracle_mod.ar_residual_rmsnorm([host_np(p) for p in parts], host_np(res),
                                                      gam.numpy(), 1e-6, "bf16")
    assert_bit_exact(host_np(o["ro"].cpu()), want_ro, "bf16", "residual_out")
    assert_norm_close(host_np(o["no"].cpu()), want_no, "bf16")


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_gather_is_a_bit_exact_copy(oracle_mod, dtype):
    """Arbitrary bit patterns (NaN payloads, subnormals, -0) come through unchanged, and no byte
    outside `out` is written."""
    W, M, H = 8, 37, 1024
    gen = torch.Generator().manual_seed(9)
    itype = torch.int32 if dtype == "fp32" else torch.int16
    tdt = synth.TORCH_DTYPES[dtype]
    slices, host = [], []
    for j in range(W):
        b, c = ar.ar_row_partition(W, M, j)
        raw = torch.randint(-2 ** 15, 2 ** 15, (c, H), generator=gen, dtype=torch.int32)
        if dtype == "fp32":
            raw = raw * 65536 + torch.randint(0, 2 ** 16, (c, H), generator=gen, dtype=torch.int32)
        raw = raw.to(itype)
        host.append(raw.numpy())
        slices.append(raw.view(tdt).cuda())
    guard = 512
    canary = 0x5A5A if itype == torch.int16 else 0x5A5A5A5A
    buf = torch.full((guard + M * H + guard,), canary, dtype=itype, device="cuda")
    out = buf[guard:guard + M * H].view(tdt).view(M, H)
    ar.ar_all_gather(slices, out)
    torch.cuda.synchronize()
    got = out.view(itype).cpu().numpy()
    assert np.array_equal(got, oracle_mod.all_gather(host))
    b = buf.cpu().numpy()
    assert (b[:guard] == canary).all() and (b[guard + M * H:] == canary).all()
