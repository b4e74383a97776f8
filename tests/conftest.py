import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: full-size CPU oracle work")


@pytest.fixture(scope="session")
def lib():
    """The C-ABI library through its Python binding (fails loudly if unbuilt)."""
    import gemm_group_wise_amd as uq
    return uq


def pytest_runtest_logreport(report):
    """With UQ_FAILURE_LOG set, append each failure at once (survives a crash later on)."""
    path = os.environ.get("UQ_FAILURE_LOG")
    if path and report.failed:
        with open(path, "a") as f:
            f.write(f"=== {report.nodeid} ({report.when})\n{report.longreprtext}\n\n")
