import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running")


def pytest_collection_modifyitems(config, items):
    # GPU tests run last within a session so that a CPU failure shows first.
    items.sort(key=lambda it: 1 if it.get_closest_marker("gpu") else 0)


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library on a real GPU; GPU tests fail loudly if it is missing."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test selected but no GPU is visible")
    import predictive_kv_block_amd as spin
    spin.load()          # raises if libspin.so is missing
    return spin
