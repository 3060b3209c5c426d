"""Parity at the size limits of the boundary.

* The widest rows the fused kernel accepts (AR_MAX_H_16BIT = 65536 elements for bf16/fp16,
  AR_MAX_H_FP32 = 32768 for binary32), with the launch shape the library plans, at one, eight
  and 64 partials, in the plain form and the workspace (split-row) form.
* Tensors larger than 4 GiB: element offsets past 2^31 in the flat sum (whose element-wise tail
  then also lies past that mark), the fused kernel, the two-kernel path on rows of odd width,
  the all-gather and the Lamport exchange.  Rows are independent, so sampled rows (the first
  ones, those around the 2^31-element / 4 GiB mark, the last ones) are checked against the
  oracle run on those rows alone; the gather is checked as a bit copy on the same rows.

Bar as everywhere (gpu_util): out / residual_out bit-identical, norm_out within 1 ulp (16-bit)
or 1e-5 relative (binary32).  The large inputs are drawn on the GPU by torch's seeded generator
(not by this library) and copied back only at the sampled rows.
"""
import numpy as np
import pytest
import torch

import all_reduce_residual_amd as ar
import synth
from gpu_util import assert_bit_exact, assert_norm_close, dev, host_np

pytestmark = pytest.mark.gpu

TWO31 = 1 << 31


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    ar.lib()
    yield
    torch.cuda.empty_cache()


# ---- widest rows ------------------------------------------------------------------------------

MAX_H = {"bf16": 65536, "fp16": 65536, "fp32": 32768}


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("W", [1, 8, 64])
def test_widest_rows(oracle_mod, W, dtype):
    M, H = 3, MAX_H[dtype]
    print("case widest rows W=%d M=%d H=%d %s launch %s" % (
        W, M, H, dtype, ar.ar_launch_config(ar.PATTERN_AR_RESIDUAL_RMSNORM, W, M, H,
                                            ar.dtype_code(synth.TORCH_DTYPES[dtype]))), flush=True)
    parts, res, gam = synth.custom(W, M, H, dtype, seed=900 + W)
    hp = [host_np(p) for p in parts]
    want_ro, want_no = oracle_mod.ar_residual_rmsnorm(hp, host_np(res), gam.numpy(), 1e-6, dtype)
    d_parts = [dev(p) for p in parts]
    d_res, d_gam = dev(res), dev(gam)
    for form in ("plain", "workspace"):
        ro, no = torch.empty_like(d_res), torch.empty_like(d_res)
        if form == "plain":
            ar.ar_residual_rmsnorm(d_parts, d_res, d_gam, 1e-6, ro, no)
        else:
            ws = ar.new_workspace(M, "cuda")
            ar.ar_residual_rmsnorm_ws(d_parts, d_res, d_gam, 1e-6, ro, no, ws)
        torch.cuda.synchronize()
        assert_bit_exact(host_np(ro.cpu()), want_ro, dtype, "%s residual_out" % form)
        assert_norm_close(host_np(no.cpu()), want_no, dtype, "%s norm_out" % form)


# ---- tensors past 4 GiB -----------------------------------------------------------------------

def _fill(t, g, sigma=1.0):
    """Seeded N(0, sigma) values drawn on the GPU, in slabs of rows."""
    step = max(1, (1 << 28) // t.shape[-1])
    for i in range(0, t.shape[0], step):
        t[i:i + step].normal_(0.0, sigma, generator=g)
    return t


def _big(M, H, tdt, g, sigma=1.0):
    return _fill(torch.empty((M, H), dtype=tdt, device="cuda"), g, sigma)


def _rows_at(t, rows):
    return host_np(t[torch.tensor(rows, device=t.device)].cpu())


def _sample_rows(M, H):
    """The first rows, the rows around element 2^31 (byte 4 GiB of a 16-bit tensor) and the
    last rows, in increasing order."""
    b = TWO31 // H
    rows = {0, 1, b - 1, b, b + 1, M - 2, M - 1}
    return sorted(r for r in rows if 0 <= r < M)


def test_sum_past_4gib(oracle_mod):
    """Flat sum over 2^31 + elements with a 7-element tail after the last full vector."""
    W, M, H, dtype = 2, 262401, 8191, "bf16"
    n = M * H
    assert n > TWO31 and n % 8 == 7
    print("case sum past 4 GiB W=%d M=%d H=%d n=%d" % (W, M, H, n), flush=True)
    g = torch.Generator(device="cuda")
    g.manual_seed(4101)
    parts = [_big(M, H, torch.bfloat16, g) for _ in range(W)]
    out = torch.empty_like(parts[0])
    ar.ar_sum(parts, out)
    torch.cuda.synchronize()
    flat_parts = [p.view(-1) for p in parts]
    flat_out = out.view(-1)
    for lo, hi in ((0, 4096), (TWO31 - 4096, TWO31 + 4096), (n - 4096 - 7, n)):
        want = oracle_mod.ar_sum([host_np(fp[lo:hi].cpu()).reshape(1, -1) for fp in flat_parts],
                                 dtype)
        assert_bit_exact(host_np(flat_out[lo:hi].cpu()).reshape(1, -1), want, dtype,
                         "out[%d:%d]" % (lo, hi))
    del parts, out, flat_parts, flat_out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("path", ["fused", "two_kernel"])
def test_residual_rmsnorm_past_4gib(oracle_mod, path):
    """Fused kernel at H = 7168; the two-kernel path at the odd width H = 7170 (rows that share
    16-byte vectors with their neighbours, element-wise row ends)."""
    W, M, dtype = 2, 300000, "bf16"
    H = 7168 if path == "fused" else 7170
    assert M * H > TWO31
    print("case %s past 4 GiB W=%d M=%d H=%d" % (path, W, M, H), flush=True)
    g = torch.Generator(device="cuda")
    g.manual_seed(4202 + H)
    parts = [_big(M, H, torch.bfloat16, g, 0.05) for _ in range(W)]
    res = _big(M, H, torch.bfloat16, g)
    gam = torch.empty(H, dtype=torch.float32, device="cuda").uniform_(0.5, 1.5, generator=g)
    ro, no = torch.empty_like(res), torch.empty_like(res)
    if path == "fused":
        ar.ar_residual_rmsnorm(parts, res, gam, 1e-6, ro, no)
    else:
        ar.ar_residual_rmsnorm_unfused(parts, res, gam, 1e-6, ro, no)
    torch.cuda.synchronize()
    rows = _sample_rows(M, H)
    want_ro, want_no = oracle_mod.ar_residual_rmsnorm(
        [_rows_at(p, rows) for p in parts], _rows_at(res, rows), gam.cpu().numpy(), 1e-6, dtype)
    assert_bit_exact(_rows_at(ro, rows), want_ro, dtype, "residual_out rows %s" % rows)
    assert_norm_close(_rows_at(no, rows), want_no, dtype, "norm_out rows %s" % rows)
    del parts, res, ro, no
    torch.cuda.empty_cache()


def test_all_gather_past_4gib():
    """Two slices gathered into a 4.1 GiB tensor: the second slice lands past the 4 GiB mark."""
    W, M, H = 2, 300000, 7168
    print("case all-gather past 4 GiB W=%d M=%d H=%d" % (W, M, H), flush=True)
    g = torch.Generator(device="cuda")
    g.manual_seed(4303)
    slices = []
    for j in range(W):
        _, c = ar.ar_row_partition(W, M, j)
        slices.append(_big(c, H, torch.bfloat16, g))
    out = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
    ar.ar_all_gather(slices, out)
    torch.cuda.synchronize()
    for r in _sample_rows(M, H):
        j = 0 if r < ar.ar_row_partition(W, M, 1)[0] else 1
        b, _ = ar.ar_row_partition(W, M, j)
        assert np.array_equal(_rows_at(out, [r]), _rows_at(slices[j], [r - b])), "row %d" % r
    del slices, out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("pattern", ["sum", "rms"])
def test_lamport_past_4gib(oracle_mod, pattern):
    """Receive slots of 4.1 GiB each; round 2 uses the last of the three buffers, which starts
    past 16 GiB, and its push empties buffer 0."""
    W, M, H, dtype = 2, 300000, 7168, "bf16"
    print("case lamport %s past 4 GiB W=%d M=%d H=%d" % (pattern, W, M, H), flush=True)
    g = torch.Generator(device="cuda")
    g.manual_seed(4404)
    parts = [_big(M, H, torch.bfloat16, g, 0.05) for _ in range(W)]
    rbuf = torch.empty((ar.LAMPORT_BUFFERS, W, M, H), dtype=torch.bfloat16, device="cuda")
    ar.ar_lamport_arm(rbuf)
    for r, p in enumerate(parts):
        ar.ar_lamport_push(p, r, rbuf, 2)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    rows = _sample_rows(M, H)
    hp = [_rows_at(p, rows) for p in parts]
    if pattern == "sum":
        out = torch.empty_like(parts[0])
        ar.ar_lamport_sum(rbuf, 2, out, status)
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        assert_bit_exact(_rows_at(out, rows), oracle_mod.ar_sum(hp, dtype), dtype,
                         "lamport out rows %s" % rows)
        del out
    else:
        res = _big(M, H, torch.bfloat16, g)
        gam = torch.empty(H, dtype=torch.float32, device="cuda").uniform_(0.5, 1.5, generator=g)
        ro, no = torch.empty_like(res), torch.empty_like(res)
        ar.ar_lamport_residual_rmsnorm(rbuf, 2, res, gam, 1e-6, ro, no, status)
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        want_ro, want_no = oracle_mod.ar_residual_rmsnorm(hp, _rows_at(res, rows),
                                                          gam.cpu().numpy(), 1e-6, dtype)
        assert_bit_exact(_rows_at(ro, rows), want_ro, dtype, "lamport residual_out")
        assert_norm_close(_rows_at(no, rows), want_no, dtype, "lamport norm_out")
        del res, ro, no
    # Buffer 0 was emptied by the push (all ones at the sampled rows of both slots) and buffer 2
    # holds the partials.
    iv = rbuf.view(torch.int16)
    idx = torch.tensor(rows, device="cuda")
    assert bool((iv[0][:, idx] == -1).all())
    for r, p in enumerate(parts):
        assert torch.equal(iv[2, r][idx], p.view(torch.int16)[idx])
    del parts, rbuf, iv
    torch.cuda.empty_cache()
