"""Shared pytest configuration: the ``gpu`` marker, repo-root imports and the oracle pool.

The full-size parity tests run the fp64 oracle over every token in a pool of forked CPU
processes.  The pool is forked here, when the session is configured and before any test module
is imported, so no process that has initialised the GPU ever forks.  It is started only when the
selected tests can include GPU tests (a ``-m`` expression naming ``gpu`` without ``not gpu``, or
PISA_ORACLE_POOL=1).
"""
import os
import sys

import pytest

TESTS = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(TESTS)
for path in (ROOT, TESTS):
    if path not in sys.path:
        sys.path.insert(0, path)

_POOL = {}


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP path")
    expr = (config.getoption("markexpr", "") or "").replace(" ", "")
    wants_gpu = "gpu" in expr and "notgpu" not in expr
    if wants_gpu or os.environ.get("PISA_ORACLE_POOL") == "1":
        import oracle_pool

        _POOL["pool"] = oracle_pool.make_pool()


def pytest_unconfigure(config):
    pool = _POOL.pop("pool", None)
    if pool is not None:
        pool.terminate()
        pool.join()


@pytest.fixture(scope="session")
def oracle_workers():
    """The forked oracle pool; a test that needs it fails if the session did not start one."""
    pool = _POOL.get("pool")
    if pool is None:
        pytest.fail("the oracle pool was not started: run the GPU tests with -m gpu (or PISA_ORACLE_POOL=1)")
    return pool
