import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload check (minutes of CPU work)")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library binding, on a machine with a GPU."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import mixture_experts_grouped_top_amd as moe
    moe.load()  # raises if the shared library is missing
    return moe
