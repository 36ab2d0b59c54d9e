import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def ldc():
    """The HIP path's Python binding; the library must be built and a GPU present."""
    if not gpu_available():
        pytest.skip("no GPU visible")
    import dynamic_head_composition_amd as m
    m.load_library()  # raises if the HIP library is missing: no silent fallback
    return m
