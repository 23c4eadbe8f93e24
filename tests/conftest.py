import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU test")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def ca2():
    """The HIP library binding; GPU tests fail loudly if it is missing."""
    if not gpu_available():
        pytest.fail("GPU test collected without a GPU")
    from causal_kv_cache_amd import ca2 as lib
    lib.load()
    return lib
