import multiprocessing as mp
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

_POOL = None


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running (full-size workloads)")
    # Full-size GPU parity tests build the CPU oracle's index block by block in
    # worker processes.  They are forked here, before any test touches the
    # device, and only run oracle (CPU) code.
    global _POOL
    expr = config.getoption("markexpr", "") or ""
    if "not gpu" not in expr and os.environ.get("LSA_TEST_NO_POOL") != "1":
        _POOL = mp.get_context("fork").Pool(min(16, os.cpu_count() or 1))


def pytest_unconfigure(config):
    global _POOL
    if _POOL is not None:
        _POOL.close()
        _POOL.join()
        _POOL = None


@pytest.fixture(scope="session")
def oracle_pool():
    return _POOL
