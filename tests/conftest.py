import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload (minutes of host time)")


@pytest.fixture(scope="session")
def gpu_lib():
    """The loaded HIP library; skips cleanly only when no GPU is present."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from kv_cache_int2_fwht_amd import binding
    return binding.lib()
