import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def gpu_ssd():
    """The HIP library binding; GPU tests fail loudly if it is not built or no GPU is visible."""
    import torch

    if not torch.cuda.is_available():
        pytest.fail("GPU test selected but torch sees no GPU")
    import mamba_ssd_chunked_05_amd as ssd

    ssd.load()  # raises if the shared library is missing
    return ssd
