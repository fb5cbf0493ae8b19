import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large CPU work (full-size generation)")


@pytest.fixture(scope="session")
def dg():
    """The product binding, loaded from the in-tree build; fails loudly if it is missing."""
    import fp4_gemm_dense_amd as m
    m.load_library()
    return m
