import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built libcsa2")


@pytest.fixture(scope="session")
def lib():
    """The built GPU library (fails loudly when it is missing)."""
    from fp4_kv_cache_amd import csa2
    return csa2.load()
