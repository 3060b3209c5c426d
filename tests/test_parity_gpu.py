"""Parity of the HIP path (called through the C ABI) with the CPU oracle, element by element.

Bar (written in gpu_util): out and residual_out bit-identical; norm_out within 1 ulp for
bf16/fp16 and within 1e-5 relative for fp32.  Inputs come from synth (seeded), the same arrays
go to both sides.  Covers the five workloads at their full sizes in the launch shape the
library picks (the one the benchmark times), every supported W and element type, ragged rows
and tails, every launch-shape family, the hand-derived golden fixtures and special values.
"""
import numpy as np
import pytest
import torch

import all_reduce_residual_amd as ar
import synth
from golden_fixtures import all_fixtures
from gpu_util import assert_bit_exact, assert_norm_close, dev, host_np

pytestmark = pytest.mark.gpu

TD = synth.TORCH_DTYPES


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    ar.lib()


def run_sum_both(oracle_mod, parts, dtype, config=None):
    d_parts = [dev(p) for p in parts]
    out = torch.empty_like(d_parts[0])
    ar.ar_sum(d_parts, out, config=config)
    torch.cuda.synchronize()
    want = oracle_mod.ar_sum([host_np(p) for p in parts], dtype)
    assert_bit_exact(host_np(out.cpu()), want, dtype, "out")


def run_rms_both(oracle_mod, parts, res, gam, eps, dtype, config=None, oracle_out=None):
    d_parts = [dev(p) for p in parts]
    d_res, d_gam = dev(res), dev(gam)
    ro = torch.empty_like(d_res)
    no = torch.empty_like(d_res)
    ar.ar_residual_rmsnorm(d_parts, d_res, d_gam, eps, ro, no, config=config)
    torch.cuda.synchronize()
    if oracle_out is None:
        oracle_out = oracle_mod.ar_residual_rmsnorm([host_np(p) for p in parts], host_np(res),
                                                    gam.numpy(), eps, dtype)
    want_ro, want_no = oracle_out
    assert_bit_exact(host_np(ro.cpu()), want_ro, dtype, "residual_out")
    return assert_norm_close(host_np(no.cpu()), want_no, dtype)


# ---- the five workloads at full size ---------------------------------------------------------

WL_CASES = [(name, M, pat) for name, wl in synth.WORKLOADS.items() for M in wl.Ms
            for pat in wl.patterns]


@pytest.mark.parametrize("name,M,pattern", WL_CASES,
                         ids=["%s-M%d-%s" % c for c in WL_CASES])
def test_workload_full_size(oracle_mod, name, M, pattern):
    wl = synth.WORKLOADS[name]
    print("case", name, M, pattern, flush=True)
    parts, res, gam = synth.inputs(wl, M)
    if pattern == "sum":
        run_sum_both(oracle_mod, parts, wl.dtype)
    else:
        run_rms_both(oracle_mod, parts, res, gam, wl.eps, wl.dtype)


# ---- every W x element type, ragged shapes --------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("W", [1, 2, 4, 8, 16, 32, 64])
def test_all_world_sizes(oracle_mod, dtype, W):
    M, H = 5, 1016 if dtype != "fp32" else 1012   # 127 / 253 vectors per row: ragged
    parts, res, gam = synth.custom(W, M, H, dtype, seed=1000 + W)
    run_sum_both(oracle_mod, parts, dtype)
    run_rms_both(oracle_mod, parts, res, gam, 1e-6, dtype)


RAGGED = [(1, 8), (3, 24), (2, 56), (31, 256), (33, 520), (7, 4104), (3, 8192), (2, 16384),
          (2, 32768), (1, 65536), (257, 64)]


@pytest.mark.parametrize("M,H", RAGGED, ids=["M%d-H%d" % c for c in RAGGED])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_ragged_shapes(oracle_mod, M, H, dtype):
    W = 4
    parts, res, gam = synth.custom(W, M, H, dtype, seed=M * 131 + H)
    run_sum_both(oracle_mod, parts, dtype)
    run_rms_both(oracle_mod, parts, res, gam, 1e-5, dtype)


@pytest.mark.parametrize("M,H", [(3, 13), (1, 1), (1, 7), (5, 3), (2, 1001)])
@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_sum_element_tail(oracle_mod, M, H, dtype):
    """kAllReduce accepts any M*H: the part after the last full 16-byte vector is summed
    element by element."""
    parts, _, _ = synth.custom(4, M, H, dtype, seed=7 * M + H, with_norm=False)
    run_sum_both(oracle_mod, parts, dtype)


def test_fp32_largest_row(oracle_mod):
    parts, res, gam = synth.custom(2, 2, 32768, "fp32", seed=5)
    run_rms_both(oracle_mod, parts, res, gam, 1e-6, "fp32")


# ---- every launch-shape family gives the same result ---------------------------------------

def _norm_configs(V, M):
    cfgs = []
    for vpt in (1, 2, 4, 8):
        need = -(-V // vpt)
        if need <= 64:
            lanes = 1
            while lanes < need:
                lanes *= 2
            for threads in (64, 256, 1024):
                cfgs.append(dict(threads_per_block=threads, vecs_per_thread=vpt,
                                 lanes_per_row=lanes, rows_per_block=threads // lanes,
                                 grid=max(1, min(3, M)), flat=0))
        lanes = -(-need // 64) * 64
        if lanes <= 1024:
            for grid in (1, 2, M):
                cfgs.append(dict(threads_per_block=lanes, vecs_per_thread=vpt,
                                 lanes_per_row=lanes, rows_per_block=1, grid=max(grid, 1),
                                 flat=0))
            if lanes * 2 <= 1024:
                cfgs.append(dict(threads_per_block=lanes * 2, vecs_per_thread=vpt,
                                 lanes_per_row=lanes, rows_per_block=2, grid=max(1, M // 3),
                                 flat=0))
    return cfgs


@pytest.mark.parametrize("H", [64, 256, 1016, 7168])
def test_norm_launch_shapes_agree(oracle_mod, H):
    dtype, M, W = "bf16", 9, 8
    parts, res, gam = synth.custom(W, M, H, dtype, seed=H)
    want = oracle_mod.ar_residual_rmsnorm([host_np(p) for p in parts], host_np(res),
                                          gam.numpy(), 1e-6, dtype)
    cfgs = _norm_configs(H // 8, M)
    assert len(cfgs) >= 4
    for i, cfg in enumerate(cfgs):
        cfg["nt_store"] = i % 2          # both store policies
        run_rms_both(oracle_mod, parts, res, gam, 1e-6, dtype, config=cfg, oracle_out=want)


def _rank_batch_built(W, vpt, n):
    """The fixed rank batches the library is built with (the launch checks allow these only)."""
    return ((n == 1 and ((vpt == 2 and 4 <= W <= 16) or (vpt == 4 and W in (2, 4)))) or
            (n == 2 and ((vpt == 2 and W >= 4) or (vpt == 1 and W >= 32))) or
            (n == 4 and vpt == 2 and W == 8))


# Ragged rows: 250 vectors (H = 2000 at 16 bits, 1000 in binary32) over 128 lanes x 2 or 256 x 1,
# and 255 / 510 vectors (H = 2040) over 64 / 128 lanes x 4.
RANK_CASES = [(W, H if dtype != "fp32" or vpt == 4 else H // 2, dtype, vpt, n)
              for W in (2, 4, 8, 16, 32, 64) for dtype in ("bf16", "fp16", "fp32")
              for H, vpt in ((2000, 1), (2000, 2), (2040, 4)) for n in (1, 2, 4)
              if _rank_batch_built(W, vpt, n)]


@pytest.mark.parametrize("W,H,dtype,vpt,n", RANK_CASES,
                         ids=["W%d-H%d-%s-v%d-r%d" % c for c in RANK_CASES])
def test_rank_batch_shapes_agree(oracle_mod, W, H, dtype, vpt, n):
    """Fixed rank batches (one rank per batch at one to three rows per CU, two or four beyond)
    give the oracle's result: one and two rows per block, a ragged row (lanes past its last
    vector), grid stride."""
    M = 13
    parts, res, gam = synth.custom(W, M, H, dtype, seed=W * 7 + H + vpt + 1000 * n)
    want = oracle_mod.ar_residual_rmsnorm([host_np(p) for p in parts], host_np(res),
                                          gam.numpy(), 1e-6, dtype)
    V = H * (4 if dtype == "fp32" else 2) // 16
    lanes = -(-(-(-V // vpt)) // 64) * 64
    for rows, grid in ((1, M), (1, 4), (2, 3)):
        if lanes * rows > 1024:
            continue
        cfg = dict(threads_per_block=lanes * rows, vecs_per_thread=vpt, lanes_per_row=lanes,
                   rows_per_block=rows, grid=grid, flat=0, nt_store=1, ranks_per_batch=n)
        print("case rank batch", W, H, dtype, cfg, flush=True)
        run_rms_both(oracle_mod, parts, res, gam, 1e-6, dtype, config=cfg, oracle_out=want)


def test_planned_rank_batch_workloads(oracle_mod):
    """The planned shapes around the band edges: one rank per batch at two and three rows per CU,
    four ranks just past three rows per CU (the wide-hidden call, W = 8 H = 7168 bf16), against
    the oracle on every row."""
    cu = ar.ar_device_cu_count()
    for M, n in ((2 * cu, 1), (3 * cu, 1), (3 * cu + 1, 4)):
        assert ar.ar_launch_config(ar.PATTERN_AR_RESIDUAL_RMSNORM, 8, M, 7168,
                                   ar.DTYPE_BF16)["ranks_per_batch"] == n
        print("case planned rank batch M=%d n=%d" % (M, n), flush=True)
        parts, res, gam = synth.inputs(synth.WORKLOADS["wide_hidden"], M)
        run_rms_both(oracle_mod, parts, res, gam, 1e-6, "bf16")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_sum_launch_shapes_agree(oracle_mod, dtype):
    parts, _, _ = synth.custom(8, 37, 1000, dtype, seed=77, with_norm=False)
    for threads in (64, 256, 1024):
        for u in (1, 2, 4):
            for grid in (1, 7, 10000):
                run_sum_both(oracle_mod, parts, dtype,
                             config=dict(threads_per_block=threads, vecs_per_thread=u,
                                         lanes_per_row=0, rows_per_block=0, grid=grid, flat=1,
                                         nt_store=(threads + u + grid) % 2))


# ---- hand-derived golden fixtures --------------------------------------------------------------

FIXTURES = all_fixtures()


def _from_storage(a: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "fp32":
        return torch.from_numpy(a.copy())
    return torch.from_numpy(a.view(np.int16).copy()).view(TD[dtype])


@pytest.mark.parametrize("fx", FIXTURES, ids=[f["name"] for f in FIXTURES])
def test_golden_fixtures_on_gpu(fx):
    dt = fx["dtype"]
    parts = [dev(_from_storage(x, dt)) for x in fx["inputs"]]
    if fx["pattern"] == "sum":
        out = torch.empty_like(parts[0])
        ar.ar_sum(parts, out)
        assert_bit_exact(host_np(out.cpu()), fx["out"], dt, "out")
    else:
        res = dev(_from_storage(fx["residual"], dt))
        gam = dev(torch.from_numpy(fx["gamma"]))
        ro, no = torch.empty_like(res), torch.empty_like(res)
        ar.ar_residual_rmsnorm(parts, res, gam, fx["eps"], ro, no)
        assert_bit_exact(host_np(ro.cpu()), fx["residual_out"], dt, "residual_out")
        assert_bit_exact(host_np(no.cpu()), fx["norm_out"], dt, "norm_out")


# ---- special values ------------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_special_values(oracle_mod, dtype):
    """Subnormals, signed zeros, overflow to infinity, infinities and NaN in the partials."""
    M, H, W = 4, 64, 4
    rng = np.random.default_rng(3)
    if dtype == "fp32":
        pool = np.array([0.0, -0.0, 1e-45, -1e-45, 1.1754942e-38, 3.4e38, -3.4e38, np.inf,
                         -np.inf, np.nan, 1.0, -2.5, 65504.0], dtype=np.float32)
        parts = [torch.from_numpy(rng.choice(pool, size=(M, H)).astype(np.float32))
                 for _ in range(W)]
    else:
        if dtype == "fp16":
            pool = [0x0000, 0x8000, 0x0001, 0x8001, 0x03FF, 0x0400, 0x7BFF, 0xFBFF, 0x7C00,
                    0xFC00, 0x7E00, 0x3C00, 0xC100]
        else:
            pool = [0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x0080, 0x7F7F, 0xFF7F, 0x7F80,
                    0xFF80, 0x7FC0, 0x3F80, 0xC020]
        parts = [torch.from_numpy(rng.choice(np.array(pool, dtype=np.uint16), size=(M, H))
                                  .view(np.int16)).view(TD[dtype]) for _ in range(W)]
    run_sum_both(oracle_mod, parts, dtype)
    res = torch.zeros(M, H, dtype=TD[dtype])
    gam = torch.ones(H, dtype=torch.float32)
    run_rms_both(oracle_mod, parts, res, gam, 1e-6, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_subnormal_results_kept(oracle_mod, dtype):
    """Cancellation into the subnormal range of T: no flush to zero on either side."""
    M, H = 2, 256
    tiny = {"fp16": 2.0 ** -20, "bf16": 2.0 ** -130}[dtype]
    x0 = torch.full((M, H), 3 * tiny, dtype=torch.float32)
    x1 = torch.full((M, H), -2 * tiny, dtype=torch.float32)
    parts = [x0.to(TD[dtype]), x1.to(TD[dtype])]
    run_sum_both(oracle_mod, parts, dtype)


def test_fp16_outliers_cancel(oracle_mod):
    """+-50 outliers over 16 ranks (the many-rank fp16 workload's distribution) at a small
    shape: cancellation makes the rank order visible in the last bits."""
    wl = synth.WORKLOADS["fp16_many_rank"]
    parts = [synth.partial(wl, r, 6) for r in range(wl.W)]
    run_sum_both(oracle_mod, parts, "fp16")


# ---- launch shapes the planner picks for one or two partials at large M -------------------------

@pytest.mark.parametrize("W,M,H", [(2, 2048, 4096), (2, 1024, 8192), (1, 2048, 7168), (1, 600, 4096),
                                   (2, 600, 4096)])
def test_small_world_planned_shapes(oracle_mod, W, M, H):
    """More rows than CUs with W <= 2: the planner shrinks the row block (down to one wave with
    8 vectors per thread); the result is the oracle's."""
    cfg = ar.ar_launch_config(ar.PATTERN_AR_RESIDUAL_RMSNORM, W, M, H, ar.DTYPE_BF16)
    print("case", W, M, H, cfg, flush=True)
    parts, res, gam = synth.custom(W, M, H, "bf16", seed=W * 100 + M + H)
    run_rms_both(oracle_mod, parts, res, gam, 1e-6, "bf16")


@pytest.mark.parametrize("W", [1, 2, 4, 8, 16, 32, 64])
@pytest.mark.parametrize("vpt", [4, 8])
@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_norm_vectors_per_thread_branches(oracle_mod, W, vpt, dtype):
    """4 and 8 vectors per thread take the all-chains branch when (W + 1) x vpt <= 20 and the
    grouped branch otherwise (groups of 4, 2 or 1 vectors, staged for groups of 2 or more,
    the 16-rank walk at W >= 32); every branch matches the oracle, with ragged rows."""
    M, H = 37, 4096 - 8 if dtype != "fp32" else 4096 - 4
    V = H // (8 if dtype != "fp32" else 4)
    lanes = -(-(-(-V // vpt)) // 64) * 64
    cfg = dict(threads_per_block=lanes, vecs_per_thread=vpt, lanes_per_row=lanes,
               rows_per_block=1, grid=M, flat=0, nt_store=1)
    parts, res, gam = synth.custom(W, M, H, dtype, seed=W * 10 + vpt)
    run_rms_both(oracle_mod, parts, res, gam, 1e-6, dtype, config=cfg)


# ---- the sum's one-round launch shapes at every world size ----------------------------------------

ROUND_CASES = [(2, 128, 7168, "bf16"), (4, 128, 7168, "bf16"), (4, 127, 7169, "bf16"),
               (2, 64, 7168, "bf16"), (8, 511, 7169, "bf16"), (16, 512, 7168, "bf16"),
               (32, 512, 7168, "bf16"), (64, 512, 7168, "bf16"), (16, 512, 8192, "bf16"),
               (64, 450, 7173, "bf16"), (4, 64, 7168, "fp32"), (8, 256, 7168, "fp32"),
               (32, 255, 7171, "fp32"), (2, 100, 7170, "fp16"), (16, 512, 8192, "fp16"),
               (16, 1024, 8192, "bf16"), (32, 600, 7173, "fp16")]


@pytest.mark.parametrize("W,M,H,dtype", ROUND_CASES,
                         ids=["W%d-M%d-H%d-%s" % c for c in ROUND_CASES])
def test_sum_resident_round_shapes(oracle_mod, W, M, H, dtype):
    """Sizes that the planner covers with 256-thread blocks (one vector per thread for W <= 8
    in one resident round, four for W >= 8 up to 2 or, from 16 ranks, 8 blocks per CU), odd
    widths leaving an element-wise tail; the whole output against the oracle.  Inputs are
    drawn on the GPU by torch's seeded generator."""
    tdt = TD[dtype]
    cfg = ar.ar_launch_config(ar.PATTERN_ALLREDUCE, W, M, H, ar.dtype_code(tdt))
    print("case", W, M, H, dtype, cfg, flush=True)
    assert cfg["threads_per_block"] == 256 and cfg["vecs_per_thread"] in (1, 4)
    g = torch.Generator(device="cuda")
    g.manual_seed(W * 1000 + M)
    parts = [torch.empty((M, H), dtype=tdt, device="cuda").normal_(0.0, 1.0, generator=g)
             for _ in range(W)]
    out = torch.empty_like(parts[0])
    ar.ar_sum(parts, out)
    torch.cuda.synchronize()
    want = oracle_mod.ar_sum([host_np(p.cpu()) for p in parts], dtype)
    assert_bit_exact(host_np(out.cpu()), want, dtype, "out")


SINGLE_WAVE = [(8, 256, 7168, "bf16"), (4, 160, 7171, "bf16"), (2, 200, 7168, "fp16"),
               (8, 128, 7168, "fp32"), (8, 16, 7168, "bf16"), (4, 20, 7170, "fp32")]


@pytest.mark.parametrize("W,M,H,dtype", SINGLE_WAVE,
                         ids=["W%d-M%d-H%d-%s" % c for c in SINGLE_WAVE])
def test_sum_single_wave_shapes(oracle_mod, W, M, H, dtype):
    """Sizes the planner covers with single-wave blocks: one vector per thread from 8 blocks per
    CU, two below (the last two cases), odd widths with an element-wise tail; whole output."""
    tdt = TD[dtype]
    cfg = ar.ar_launch_config(ar.PATTERN_ALLREDUCE, W, M, H, ar.dtype_code(tdt))
    print("case", W, M, H, dtype, cfg, flush=True)
    assert cfg["threads_per_block"] == 64
    assert cfg["vecs_per_thread"] == (2 if M <= 20 else 1)
    parts, _, _ = synth.custom(W, M, H, dtype, seed=W * 101 + M, with_norm=False)
    run_sum_both(oracle_mod, parts, dtype)

# ---- many ranks at many rows: one vector per thread over the whole row -----------------------------

MANY = [(32, 2048, 7168, "bf16"), (64, 2048, 8192, "fp16")]


@pytest.mark.parametrize("W,M,H,dtype", MANY, ids=["W%d-M%d-H%d-%s" % c for c in MANY])
def test_many_ranks_many_rows_sampled(oracle_mod, W, M, H, dtype):
    """The planned shape for W >= 32 with 16-bit rows and >= 8 rows per CU; sampled rows of
    both outputs against the oracle run on those rows.  Inputs drawn on the GPU by torch's
    seeded generator."""
    tdt = TD[dtype]
    cfg = ar.ar_launch_config(ar.PATTERN_AR_RESIDUAL_RMSNORM, W, M, H, ar.dtype_code(tdt))
    print("case", W, M, H, dtype, cfg, flush=True)
    assert cfg["vecs_per_thread"] == 1 and cfg["lanes_per_row"] * 8 == H
    g = torch.Generator(device="cuda")
    g.manual_seed(W + M)
    parts = [torch.empty((M, H), dtype=tdt, device="cuda").normal_(0.0, 0.05, generator=g)
             for _ in range(W)]
    res = torch.empty((M, H), dtype=tdt, device="cuda").normal_(0.0, 1.0, generator=g)
    gam = torch.empty(H, dtype=torch.float32, device="cuda").uniform_(0.5, 1.5, generator=g)
    ro, no = torch.empty_like(res), torch.empty_like(res)
    ar.ar_residual_rmsnorm(parts, res, gam, 1e-6, ro, no)
    torch.cuda.synchronize()
    rows = torch.tensor([0, 1, 255, 256, 1023, 1024, M - 2, M - 1], device="cuda")
    want_ro, want_no = oracle_mod.ar_residual_rmsnorm(
        [host_np(p[rows].cpu()) for p in parts], host_np(res[rows].cpu()),
        gam.cpu().numpy(), 1e-6, dtype)
    assert_bit_exact(host_np(ro[rows].cpu()), want_ro, dtype, "residual_out")
    assert_norm_close(host_np(no[rows].cpu()), want_no, dtype)


# ---- planned rank batches at prefill sizes (more than three rows per CU) ------------------------

PREFILL_BATCHES = [(4, 2048, 7168, "bf16", 2, 2), (8, 2048, 8192, "fp16", 2, 4),
                   (8, 2048, 4096, "fp32", 2, 2), (16, 2048, 7168, "bf16", 2, 2),
                   (32, 1024, 7168, "bf16", 2, 2), (64, 2048, 2048, "fp32", 1, 2)]


@pytest.mark.parametrize("W,M,H,dtype,vpt,n", PREFILL_BATCHES,
                         ids=["W%d-M%d-H%d-%s" % c[:4] for c in PREFILL_BATCHES])
def test_planned_rank_batches_sampled(oracle_mod, W, M, H, dtype, vpt, n):
    """The planned shapes that load two or four ranks per batch beyond three rows per CU: sampled
    rows of both outputs against the oracle run on those rows (inputs drawn on the GPU by
    torch's seeded generator)."""
    tdt = TD[dtype]
    cu = ar.ar_device_cu_count()
    cfg = ar.ar_launch_config(ar.PATTERN_AR_RESIDUAL_RMSNORM, W, M, H, ar.dtype_code(tdt))
    print("case", W, M, H, dtype, cfg, flush=True)
    if M <= 3 * cu or (vpt == 1 and M < 8 * cu):
        pytest.skip("rows per CU on this device fall outside the band")
    assert cfg["vecs_per_thread"] == vpt and cfg["ranks_per_batch"] == n, cfg
    g = torch.Generator(device="cuda")
    g.manual_seed(W * 7 + M)
    parts = [torch.empty((M, H), dtype=tdt, device="cuda").normal_(0.0, 0.05, generator=g)
             for _ in range(W)]
    res = torch.empty((M, H), dtype=tdt, device="cuda").normal_(0.0, 1.0, generator=g)
    gam = torch.empty(H, dtype=torch.float32, device="cuda").uniform_(0.5, 1.5, generator=g)
    ro, no = torch.empty_like(res), torch.empty_like(res)
    ar.ar_residual_rmsnorm(parts, res, gam, 1e-6, ro, no)
    torch.cuda.synchronize()
    rows = torch.tensor(sorted({0, 1, 255, 256, 767, 768, M // 2, M - 2, M - 1}), device="cuda")
    want_ro, want_no = oracle_mod.ar_residual_rmsnorm(
        [host_np(p[rows].cpu()) for p in parts], host_np(res[rows].cpu()),
        gam.cpu().numpy(), 1e-6, dtype)
    assert_bit_exact(host_np(ro[rows].cpu()), want_ro, dtype, "residual_out")
    assert_norm_close(host_np(no[rows].cpu()), want_no, dtype)


# ---- seeded random shapes through every entry point, in the launch shapes the library picks -----

def _random_cases(n=36, seed=20261202):
    """(W, M, H, dtype) drawn from a fixed seed: every supported W and type, M log-uniform over
    1 ... 1536 rows, H any whole number of 16-byte vectors up to the type's limit, capped at
    6 Mi summed elements so the oracle stays quick."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        W = int(rng.choice([1, 2, 4, 8, 16, 32, 64]))
        dtype = str(rng.choice(["bf16", "fp16", "fp32"]))
        vec = 4 if dtype == "fp32" else 8
        max_v = (32768 if dtype == "fp32" else 65536) // vec
        V = int(np.exp(rng.uniform(0.0, np.log(max_v))))
        M = int(np.exp(rng.uniform(0.0, np.log(1536))))
        H = max(1, V) * vec
        if (W + 1) * M * H > 6 << 20:
            continue
        cases.append((W, M, H, dtype))
    return cases


RANDOM = _random_cases()


@pytest.mark.parametrize("W,M,H,dtype", RANDOM, ids=["W%d-M%d-H%d-%s" % c for c in RANDOM])
def test_random_shapes_every_entry_point(oracle_mod, W, M, H, dtype):
    """ar_sum, ar_residual_rmsnorm, its workspace form and its two-kernel form, each in the launch
    shape the library plans for the shape, against one oracle result."""
    print("case", W, M, H, dtype, flush=True)
    parts, res, gam = synth.custom(W, M, H, dtype, seed=W * 7919 + M * 31 + H)
    d_parts = [dev(p) for p in parts]
    d_res, d_gam = dev(res), dev(gam)
    h_parts = [host_np(p) for p in parts]
    want_out = oracle_mod.ar_sum(h_parts, dtype)
    want_ro, want_no = oracle_mod.ar_residual_rmsnorm(h_parts, host_np(res), gam.numpy(), 1e-6,
                                                      dtype)
    out = torch.empty_like(d_res)
    ar.ar_sum(d_parts, out)
    ws = ar.new_workspace(M, "cuda")
    forms = {"fused": lambda ro, no: ar.ar_residual_rmsnorm(d_parts, d_res, d_gam, 1e-6, ro, no),
             "workspace": lambda ro, no: ar.ar_residual_rmsnorm_ws(d_parts, d_res, d_gam, 1e-6,
                                                                   ro, no, ws),
             "two-kernel": lambda ro, no: ar.ar_residual_rmsnorm_unfused(d_parts, d_res, d_gam,
                                                                         1e-6, ro, no)}
    got = {}
    for name, call in forms.items():
        ro, no = torch.empty_like(d_res), torch.empty_like(d_res)
        call(ro, no)
        got[name] = (ro, no)
    torch.cuda.synchronize()
    assert_bit_exact(host_np(out.cpu()), want_out, dtype, "out")
    for name, (ro, no) in got.items():
        assert_bit_exact(host_np(ro.cpu()), want_ro, dtype, name + " residual_out")
        assert_norm_close(host_np(no.cpu()), want_no, dtype, name + " norm_out")


# ---- binary32 rows of 1025-2048 vectors: two vectors per thread at few or many rows ---------------

F32_ROWS = [(8, 1, 7168), (32, 64, 7168), (64, 16, 5120), (2, 40, 8192), (8, 2048, 7168),
            (2, 2048, 8192)]


@pytest.mark.parametrize("W,M,H", F32_ROWS, ids=["W%d-M%d-H%d" % c for c in F32_ROWS])
def test_binary32_two_vector_rows(oracle_mod, W, M, H):
    """The planned shape (up to 1024 lanes, two vectors per thread) against the oracle: every row
    at few rows, sampled rows at 2048 (inputs drawn on the GPU by torch's seeded generator)."""
    cfg = ar.ar_launch_config(ar.PATTERN_AR_RESIDUAL_RMSNORM, W, M, H, ar.dtype_code(torch.float32))
    print("case", W, M, H, cfg, flush=True)
    assert cfg["vecs_per_thread"] == 2 and cfg["lanes_per_row"] * 8 >= H
    if M < 2048:
        parts, res, gam = synth.custom(W, M, H, "fp32", seed=W * 17 + M + H)
        run_rms_both(oracle_mod, parts, res, gam, 1e-6, "fp32")
        return
    g = torch.Generator(device="cuda")
    g.manual_seed(W * 3 + M)
    parts = [torch.empty((M, H), dtype=torch.float32, device="cuda").normal_(0.0, 1.0, generator=g)
             for _ in range(W)]
    res = torch.empty((M, H), dtype=torch.float32, device="cuda").normal_(0.0, 1.0, generator=g)
    gam = torch.empty(H, dtype=torch.float32, device="cuda").uniform_(0.5, 1.5, generator=g)
    ro, no = torch.empty_like(res), torch.empty_like(res)
    ar.ar_residual_rmsnorm(parts, res, gam, 1e-6, ro, no)
    torch.cuda.synchronize()
    rows = torch.tensor([0, 1, 255, 256, 1023, 1024, M - 2, M - 1], device="cuda")
    want_ro, want_no = oracle_mod.ar_residual_rmsnorm(
        [host_np(p[rows].cpu()) for p in parts], host_np(res[rows].cpu()),
        gam.cpu().numpy(), 1e-6, "fp32")
    assert_bit_exact(host_np(ro[rows].cpu()), want_ro, "fp32", "residual_out")
    assert_norm_close(host_np(no[rows].cpu()), want_no, "fp32")


# ---- eight or more partials on rows of over 2048 vectors: four vectors per thread -------------

WIDE_MANY = [(16, 3, 20480, "fp16"), (16, 2, 32768, "bf16"), (32, 2, 24576, "bf16"),
             (64, 2, 20480, "bf16"), (8, 5, 20480, "bf16"), (16, 300, 20480, "bf16"),
             (16, 3, 12288, "fp32"), (32, 1, 10240, "fp32")]


@pytest.mark.parametrize("W,M,H,dtype", WIDE_MANY, ids=["W%d-M%d-H%d-%s" % c for c in WIDE_MANY])
def test_many_partials_widest_rows(oracle_mod, W, M, H, dtype):
    """The planned 4-vector shape on rows of 2560-4096 vectors, whole output against the
    oracle."""
    cfg = ar.ar_launch_config(ar.PATTERN_AR_RESIDUAL_RMSNORM, W, M, H, ar.dtype_code(TD[dtype]))
    print("case", W, M, H, dtype, cfg, flush=True)
    assert cfg["vecs_per_thread"] == 4
    parts, res, gam = synth.custom(W, M, H, dtype, seed=W * 13 + M + H)
    run_rms_both(oracle_mod, parts, res, gam, 1e-6, dtype)
