import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_addoption(parser):
    parser.addoption("--margins-dir", default=None,
                     help="write the full-size parity tests' worst row errors here as JSON")


_blas_limit = None


def pytest_configure(config):
    # The oracle's matrix products are small (one token at a time): BLAS
    # threads only add synchronization (measured 20x slower with 8 threads
    # than with one), so the test process keeps BLAS on one thread.
    global _blas_limit
    import numpy  # noqa: F401  (load BLAS first: the limit applies to loaded libraries)
    from threadpoolctl import threadpool_limits
    _blas_limit = threadpool_limits(limits=1, user_api="blas")
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session")
def root():
    return ROOT
