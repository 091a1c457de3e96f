import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs a ROCm GPU (MI355X / gfx950) and the built HIP library")


def gpu_available() -> bool:
    try:
        import torch
    except Exception:
        return False
    return torch.cuda.is_available()


@pytest.fixture(scope="session")
def lib():
    """The Python binding over the C-ABI library (HIP path)."""
    if not gpu_available():
        pytest.skip("no GPU visible")
    import dequant_backward_gemm_amd as nb
    return nb
