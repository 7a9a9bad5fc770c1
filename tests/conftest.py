import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.dirname(os.path.abspath(__file__))
for p in (ROOT, HERE):
    if p not in sys.path:
        sys.path.insert(0, p)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_sessionstart(session):
    # GPU runs compare whole batches against the oracle in worker processes: start them now,
    # before any test initialises the GPU, so no worker is forked from a process holding GPU
    # state
    expr = session.config.getoption("markexpr") or ""
    if "gpu" in expr and "not gpu" not in expr:
        import oracle_pool
        oracle_pool.pool()


def pytest_collection_modifyitems(config, items):
    # GPU tests fail loudly (not skip) when selected with -m gpu on a machine without a GPU;
    # when not selected they are deselected by the marker expression.
    pass
