import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU test (skipped unless ATTN_SLOW_TESTS=1)")


def pytest_collection_modifyitems(config, items):
    if os.environ.get("ATTN_SLOW_TESTS") == "1":
        return
    skip = pytest.mark.skip(reason="slow; set ATTN_SLOW_TESTS=1")
    for it in items:
        if "slow" in it.keywords:
            it.add_marker(skip)


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.build()  # always rebuild: the .so is not committed
    oracle._lib = None
    oracle.lib()
    return oracle
