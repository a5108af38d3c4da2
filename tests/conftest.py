import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU case")


@pytest.fixture(scope="session")
def gpu():
    """Skip unless a GPU is present; returns the loaded HIP binding."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import invariant_bi_gemm_02_amd as bi
    bi.load()  # raises if the HIP library is missing: no fallback path exists
    return bi
