import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload (seconds to a minute)")


def gpu_available() -> bool:
    try:
        import torch
    except Exception:
        return False
    return bool(torch.cuda.is_available())


@pytest.fixture(scope="session")
def lib():
    """The built HIP library through its Python binding (GPU tests only)."""
    if not gpu_available():
        pytest.skip("no GPU visible")
    import int8_quantized_matmul_col_amd as mm
    mm.load()  # raises if the shared library is missing: no fallback exists
    return mm
