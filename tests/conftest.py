"""Shared pytest configuration.

Markers: ``gpu`` marks tests that need an MI355X (they call the HIP library through its C ABI);
everything else runs on the host.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs a GPU (MI355X); calls the HIP library")


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle
    oracle.build(force=False)
    return oracle
