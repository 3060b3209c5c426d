"""The README's Python examples, run as written there, with their results checked against the
oracle (sampled rows of the wide-hidden call; every row of the 8-token workspace call)."""
import pytest
import torch

import all_reduce_residual_amd as ar
from gpu_util import assert_bit_exact, assert_norm_close, host_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    ar.lib()


def test_readme_examples(oracle_mod):
    print("case readme examples W=8 M=2048 H=7168 bf16", flush=True)
    torch.manual_seed(0)
    parts = [torch.randn(2048, 7168, device="cuda").bfloat16() for _ in range(8)]
    res = torch.randn(2048, 7168, device="cuda").bfloat16()
    gamma = torch.ones(7168, device="cuda")
    ro, no = torch.empty_like(res), torch.empty_like(res)
    ar.ar_residual_rmsnorm(parts, res, gamma, 1e-6, ro, no)
    out = torch.empty_like(res)
    ar.ar_sum(parts, out)
    ws = ar.new_workspace(64, "cuda")
    p8 = [p[:8] for p in parts]
    ro8, no8 = torch.empty_like(res[:8]), torch.empty_like(res[:8])
    ar.ar_residual_rmsnorm_ws(p8, res[:8], gamma, 1e-6, ro8, no8, ws)
    torch.cuda.synchronize()

    rows = (1020, 1030)
    sl = slice(*rows)
    hp = [host_np(p) for p in parts]
    g = gamma.cpu().numpy()
    want_ro, want_no = oracle_mod.ar_residual_rmsnorm(hp, host_np(res), g, 1e-6, "bf16", rows=rows)
    assert_bit_exact(host_np(ro)[sl], want_ro[sl], "bf16", "residual_out")
    assert_norm_close(host_np(no)[sl], want_no[sl], "bf16")
    assert_bit_exact(host_np(out)[sl], oracle_mod.ar_sum(hp, "bf16", rows=rows)[sl], "bf16", "sum")
    w_ro8, w_no8 = oracle_mod.ar_residual_rmsnorm([h[:8] for h in hp], host_np(res)[:8], g, 1e-6,
                                                  "bf16")
    assert_bit_exact(host_np(ro8), w_ro8, "bf16", "workspace residual_out")
    assert_norm_close(host_np(no8), w_no8, "bf16", "workspace norm_out")

    # The routed call: at this size the default policy takes rank 0's two-shot share.
    route = ar.ar_allreduce_routed(parts, ro, residual=res, gamma=gamma, eps=1e-6, norm_out=no,
                                   rank=0)
    assert route == ar.ROUTE_TWO_SHOT

    rbuf = torch.empty((3, 8, 2048, 7168), dtype=torch.bfloat16, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    ar.ar_lamport_arm(rbuf)
    for k in range(4):
        for r in range(8):
            ar.ar_lamport_push(parts[r], r, rbuf, k)
        ar.ar_lamport_residual_rmsnorm(rbuf, k, res, gamma, 1e-6, ro, no, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert_bit_exact(host_np(ro)[sl], want_ro[sl], "bf16", "Lamport residual_out")
    assert_norm_close(host_np(no)[sl], want_no[sl], "bf16", "Lamport norm_out")
