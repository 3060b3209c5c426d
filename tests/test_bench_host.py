"""Host logic of bench.py (no GPU): the metric's byte count and the summaries it writes from
rocprofv3 output."""
import csv
import json
import os

import bench


def test_metric_bytes():
    # kARResidualRMSNorm: W partial reads + residual read + two writes; kAllReduce: W reads + 1.
    assert bench.metric_bytes("rms", 8, 2048, 7168, 2) == 322_961_408
    assert bench.metric_bytes("rms_ws", 8, 2048, 7168, 2) == 322_961_408
    assert bench.metric_bytes("unfused", 8, 2048, 7168, 2) == 322_961_408
    assert bench.metric_bytes("sum", 8, 2048, 7168, 2) == 264_241_152
    assert bench.metric_bytes("sum", 4, 5120, 8192, 2) == 419_430_400
    assert bench.metric_bytes("rmsnorm", 1, 2048, 7168, 2) == 2 * 2048 * 7168 * 2


def _trace(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Workgroup_Size_X", "Grid_Size_X",
                                          "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_sweep_trace_summary(tmp_path):
    """One-block rows (M = grid / block), split rows (M = grid / block / segments) and flat sums
    (M = grid x U / vectors per row) are attributed to their sweep entries."""
    norm = "void arf::ar_norm_kernel<arf::Bf16, 8, 2, true, arf::StreamSource, false>(...)"
    split = "void arf::ar_norm_split_kernel<arf::Bf16, 8, 1, true>(...)"
    summ = "void arf::ar_sum_kernel<arf::Bf16, 8, 2, true, arf::StreamSource>(...)"
    rows = []
    for i in range(3):
        rows.append(dict(Kernel_Name=norm, Workgroup_Size_X=448, Grid_Size_X=448 * 32,
                         Start_Timestamp=1000 * i, End_Timestamp=1000 * i + 3000))
        # 32 rows x 7 segments of 128 lanes (896 vectors per row).
        rows.append(dict(Kernel_Name=split, Workgroup_Size_X=128, Grid_Size_X=128 * 7 * 32,
                         Start_Timestamp=1000 * i, End_Timestamp=1000 * i + 2000))
        # 32 rows x 896 vectors / 2 per thread.
        rows.append(dict(Kernel_Name=summ, Workgroup_Size_X=64, Grid_Size_X=32 * 896 // 2,
                         Start_Timestamp=0, End_Timestamp=1500))
    d = tmp_path / "trace"
    d.mkdir()
    _trace(d / "sw_kernel_trace.csv", rows)
    line = {"sweep": [
        {"pattern": "kARResidualRMSNorm", "M": 32, "bytes": 5_046_272, "us_graph": 5.3,
         "split_segments": 7, "us_graph_workspace": 4.2},
        {"pattern": "kAllReduce", "M": 32, "bytes": 4_128_768, "us_graph": 2.7}]}
    bj = tmp_path / "bench.json"
    bj.write_text("# noise\n" + json.dumps(line) + "\n")
    out = bench.summarize_sweep_trace(str(d), str(bj))
    lines = [x for x in out.splitlines() if x.startswith("| k")]
    assert len(lines) == 3, out
    by = {x.split("|")[1].strip(): x for x in lines}
    assert "| 32 | 5046272 | 3 | 3.00 |" in by["kARResidualRMSNorm"]
    assert "| 32 | 5046272 | 3 | 2.00 |" in by["kARResidualRMSNorm, split rows"]
    assert "| 4.20 |" in by["kARResidualRMSNorm, split rows"]
    assert "| 32 | 4128768 | 3 | 1.50 |" in by["kAllReduce"]
    assert os.path.exists(bj)


def _counters(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_counter_summary_scales_by_the_copy(tmp_path):
    """Counters are scaled by what they read for a copy of known size; the headline's traffic
    line and the 80 MiB sum's table come out in bytes."""
    norm = "void arf::ar_norm_kernel<arf::Bf16, 8, 2, true, arf::StreamSource, false>(...)"
    summ = "void arf::ar_sum_kernel<arf::Bf16, 4, 1, false, arf::StreamSource>(...)"
    copy = "__amd_rocclr_copyBuffer.kd"
    kib = 1024.0
    copy_fetch = bench.COPY_CAL_BYTES / 2 / kib            # the fetch counter reads half
    copy_write = bench.COPY_CAL_BYTES / kib
    norm_read, norm_write = 9 * 2048 * 7168 * 2, 2 * 2048 * 7168 * 2
    sum_read, sum_write = 4 * 5120 * 8192 * 2, 5120 * 8192 * 2
    fetch = [dict(Kernel_Name=copy, Counter_Name="FETCH_SIZE", Counter_Value=copy_fetch),
             dict(Kernel_Name=norm, Counter_Name="FETCH_SIZE", Counter_Value=norm_read / 2 / kib),
             dict(Kernel_Name=summ, Counter_Name="FETCH_SIZE", Counter_Value=sum_read / 2 / kib)]
    write = [dict(Kernel_Name=copy, Counter_Name="WRITE_SIZE", Counter_Value=copy_write),
             dict(Kernel_Name=norm, Counter_Name="WRITE_SIZE", Counter_Value=norm_write / kib),
             dict(Kernel_Name=summ, Counter_Name="WRITE_SIZE", Counter_Value=sum_write / kib)]
    fd, wd = tmp_path / "f", tmp_path / "w"
    fd.mkdir()
    wd.mkdir()
    _counters(fd / "fetch_counter_collection.csv", fetch)
    _counters(wd / "write_counter_collection.csv", write)
    out = bench.summarize_pmc(str(fd), str(wd))
    data = json.loads([x for x in out.splitlines() if x.startswith("traffic_json:")][0]
                      .split(":", 1)[1])
    assert data["traffic_bytes"] == norm_read + norm_write
    assert data["fetch_factor"] == 2.0 and data["write_factor"] == 1.0
    rows = [x for x in out.splitlines() if x.startswith("| FETCH_SIZE") or
            x.startswith("| WRITE_SIZE")]
    assert len(rows) == 4, out                            # norm and sum tables
    assert rows[2].endswith("| %d | 1.000 |" % sum_read) and "%d" % sum_read in rows[2]
    assert rows[3].endswith("| %d | 1.000 |" % sum_write)


def test_headline_parity_check_accepts_and_rejects(oracle_mod):
    """The CPU leg's spot check passes the oracle's own rows and rejects a flipped residual_out
    bit or a norm_out 2 ulp away."""
    import numpy as np
    import synth
    parts, res, gam = synth.custom(2, 3, 256, "bf16", seed=5)
    hp = [synth.storage_numpy(p) for p in parts]
    hr = synth.storage_numpy(res)
    ro, no = oracle_mod.ar_residual_rmsnorm(hp, hr, gam.numpy(), 1e-6, "bf16")
    sample = {"rows": [0, 1, 2], "eps": 1e-6, "dtype": "bf16", "parts": hp, "residual": hr,
              "gamma": gam.numpy(), "residual_out": ro.copy(), "norm_out": no.copy()}
    assert bench.check_headline_parity(sample)["norm_out_max_ulp"] == 0
    bad = dict(sample, residual_out=ro ^ np.uint16(1))
    try:
        bench.check_headline_parity(bad)
        raise RuntimeError("a flipped residual_out bit was accepted")
    except AssertionError:
        pass
    off = no.copy()
    off[1, 7] = off[1, 7] + 2 if (off[1, 7] & 0x7FFF) < 0x7F00 else off[1, 7] - 2
    try:
        bench.check_headline_parity(dict(sample, norm_out=off))
        raise RuntimeError("a norm_out 2 ulp away was accepted")
    except AssertionError:
        pass


def test_headline_windows_cover_exactly_the_timed_steps():
    for steps in (1, 3, 5, 7, 20, 200, 201):
        b = bench.headline_windows(steps)
        assert b[0] == 0 and b[-1] == steps
        assert len(b) - 1 == min(5, steps)
        lens = [b[j + 1] - b[j] for j in range(len(b) - 1)]
        assert min(lens) >= 1 and max(lens) - min(lens) <= 1
    assert bench.median([3.0, 1.0, 2.0]) == 2.0
    assert bench.median([4.0, 1.0, 2.0, 3.0]) == 2.5


def test_split_grid_covers_every_segment_once():
    """The split kernel's launch grid (bench mirrors the library's): 8 x S blocks with fewer
    than 8 rows, block (m, s) on XCD m; S x M otherwise.  Every (row, segment) gets exactly one
    block and every other block maps to a row past the last."""
    for S in (1, 2, 3, 4, 7, 14, 64):
        for M in list(range(1, 40)) + [63, 64, 65, 512, 65535, 65536]:
            gx, gy = bench.split_dims(M, S)
            if M > 4096:
                assert (gx, gy) == ((S, M) if M <= 65535 else (M * S, 1))
                continue
            seen = set()
            for y in range(gy):
                for x in range(gx):
                    if M < 8:
                        m, s = x, y
                        assert (y * gx + x) % 8 == m % 8    # linear order: XCD = id % 8
                    else:
                        m, s = y, x
                    if m < M:
                        assert s < S and (m, s) not in seen, (M, S, x, y)
                        seen.add((m, s))
            assert len(seen) == M * S, (M, S)


def test_more_than_one_gpu_is_refused():
    """--gpus N > 1 (or a multi-rank launch) exits with status 2 and says why, before touching
    a GPU."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    for argv, env in ((["--gpus", "2"], {}), (["--gpus", "1"], {"WORLD_SIZE": "2"})):
        r = subprocess.run([sys.executable, os.path.join(root, "bench.py")] + argv,
                           capture_output=True, text=True, env=dict(os.environ, **env),
                           timeout=120)
        assert r.returncode == 2, (argv, r.returncode, r.stderr)
        assert "does not run on more than one GPU" in r.stderr
