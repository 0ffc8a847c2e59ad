import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload parity (minutes)")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library and a visible GPU; GPU tests skip where there is none."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import dynamic_sparse_attention_page_amd as dsa
    return dsa
