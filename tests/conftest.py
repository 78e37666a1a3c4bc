import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs through the C-ABI library)")
    config.addinivalue_line("markers", "slow: long CPU-only check, enabled by ZERO_SLOW_TESTS=1")


def pytest_collection_modifyitems(config, items):
    if os.environ.get("ZERO_SLOW_TESTS") == "1":
        return
    skip = pytest.mark.skip(reason="slow; set ZERO_SLOW_TESTS=1")
    for item in items:
        if "slow" in item.keywords:
            item.add_marker(skip)


@pytest.fixture(scope="session")
def libzero():
    """The C-ABI library, built in-tree first if no build is present."""
    from zero_sharded_optimizer_reduce_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return _lib.load()
