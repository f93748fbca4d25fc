import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

_ORACLE_POOL = None


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.hookimpl(trylast=True)
def pytest_collection_modifyitems(session, config, items):
    """Fork the oracle's worker processes while nothing has touched the GPU yet, if a selected
    test asks for them (the -m selection has already been applied here)."""
    global _ORACLE_POOL
    if _ORACLE_POOL is None and any("oracle_pool" in getattr(it, "fixturenames", ()) for it in items):
        sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
        import oracle_pool
        _ORACLE_POOL = oracle_pool.start()


def pytest_terminal_summary(terminalreporter):
    gh = sys.modules.get("gpu_helpers")
    if gh is not None and gh.FLAT_STATS["elements"]:
        terminalreporter.write_line(f"output error, flat measures: {gh.FLAT_STATS}")
    op = sys.modules.get("oracle_pool")
    for line in (op.SUMMARIES if op is not None else []):
        terminalreporter.write_line(f"every unit: {line}")


def pytest_unconfigure(config):
    global _ORACLE_POOL
    if _ORACLE_POOL is not None:
        _ORACLE_POOL.terminate()
        _ORACLE_POOL.join()
        _ORACLE_POOL = None


@pytest.fixture(scope="session")
def oracle_pool():
    if _ORACLE_POOL is None:
        pytest.skip("the oracle worker pool is forked at collection time only")
    return _ORACLE_POOL


@pytest.fixture(scope="session")
def torch_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch
