import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: oracle work that takes more than a few seconds")


@pytest.fixture(scope="session")
def gpu():
    """Skip unless a GPU is visible; the library must then be built and loadable."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from cross_model_sparse_amd import mapflow
    mapflow.load()  # raises if the native library is missing
    return torch.device("cuda:0")
