"""The oracle reproduces every hand-derived golden fixture bit for bit (host only)."""
import numpy as np
import pytest

from golden_fixtures import all_fixtures

FIXTURES = all_fixtures()


def _bits(a):
    return a.view(np.uint32) if a.dtype == np.float32 else a


@pytest.mark.parametrize("fx", FIXTURES, ids=[f["name"] for f in FIXTURES])
def test_oracle_matches_golden(oracle_mod, fx):
    if fx["pattern"] == "sum":
        out = oracle_mod.ar_sum(fx["inputs"], fx["dtype"])
        assert np.array_equal(_bits(out), _bits(fx["out"]))
    else:
        ro, no = oracle_mod.ar_residual_rmsnorm(fx["inputs"], fx["residual"], fx["gamma"],
                                                fx["eps"], fx["dtype"])
        assert np.array_equal(_bits(ro), _bits(fx["residual_out"]))
        assert np.array_equal(_bits(no), _bits(fx["norm_out"]))


def test_fixtures_present():
    names = {f["name"] for f in FIXTURES}
    assert {"rms_bf16_exact_rows.txt", "sum_fp16_ieee_edges.txt",
            "sum_fp32_rank_order.txt"} <= names
