import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD Instinct GPU (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: large inputs (full workload sizes)")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def stdk():
    """The HIP library binding; GPU tests fail loudly if it is not built."""
    import sparse_top_decode_amd as m
    m.native.load()
    return m
