import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: slower CPU tests")


def pytest_collection_modifyitems(config, items):
    # a GPU test on a machine without a GPU is an error of the invocation, not a skip:
    # `-m gpu` is only run where torch sees the device.
    pass


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library's Python binding; fails loudly when it is not built or no GPU is seen."""
    import torch

    if not torch.cuda.is_available():
        pytest.fail("GPU test selected but torch sees no GPU")
    import mixture_experts_ffn_amd as m

    m.load_library()
    return m
