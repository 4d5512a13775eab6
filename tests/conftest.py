import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs through the HIP library)")
    config.addinivalue_line("markers", "slow: full-size workloads (minutes of host time)")


@pytest.fixture(scope="session")
def orc():
    import oracle

    return oracle


def gpu_required() -> bool:
    """With VSPMM_REQUIRE_GPU=1 (set where a GPU is expected) a missing device
    is a failure, not a skip, so a GPU job cannot pass green having tested
    nothing."""
    return os.environ.get("VSPMM_REQUIRE_GPU", "") == "1"
