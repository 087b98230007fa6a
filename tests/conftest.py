import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session")
def orc():
    from oracle import oracle
    oracle.lib()
    return oracle


def pytest_sessionstart(session):
    """Build libkvq.so (hipcc) and the C oracle (gcc) only when they are missing."""
    lib = os.path.join(ROOT, "quantized_kv_cache_07_amd", "libkvq.so")
    if not os.path.exists(lib):
        from quantized_kv_cache_07_amd import build
        build.build()
