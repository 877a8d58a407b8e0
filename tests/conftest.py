import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library through its Python binding; fails loudly when it is not there."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("gpu test collected on a machine without a GPU")
    import attention_learnable_sinks_amd as als
    als.load()  # raises when the shared library is missing
    return als
