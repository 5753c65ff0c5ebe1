import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_sessionstart(session):
    """Build the libraries in-tree if a fresh checkout has none yet (they are
    not committed).  An existing build is used as it is."""
    from gradient_reduction_optimizer_amd import build as Bd
    if any(not os.path.exists(p) for p in (Bd.LIB, Bd.PROBE_LIB, Bd.CLIENT)) and os.path.exists(Bd.HIPCC):
        Bd.build()


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def gpu():
    if not gpu_available():
        pytest.skip("no GPU visible")
    return True
