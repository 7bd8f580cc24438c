import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU test")


@pytest.fixture(scope="session")
def gpu_lib():
    """The loaded HIP library; fails (does not skip) when it is missing on a GPU run."""
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from fp8_fine_grained_act_amd import lib

    return lib
