import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the HIP library")


def pytest_collection_modifyitems(config, items):
    # Mark-based selection is done by the caller (-m gpu / -m "not gpu").
    return


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library on cuda:0; fails loudly if the GPU or the library is missing."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test selected but torch.cuda.is_available() is False")
    import mxfp8_block_scaled_08_amd as mx
    mx.load()  # raises if the shared library is absent
    return mx
