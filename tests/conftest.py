import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU test")
    # a NumPy deprecation inside the oracle would become an error in a later
    # NumPy and take every pin with it: fail on it now
    config.addinivalue_line("filterwarnings", "error::DeprecationWarning:oracle.*")


@pytest.fixture(scope="session")
def gpu_lib():
    """The loaded HIP library; the GPU tests fail (not skip) if it is missing."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from decode_attention_rdkv_amd import rdkv
    rdkv.load()
    return rdkv
