import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built libmoe")


@pytest.fixture(scope="session")
def gpu_lib():
    """The GPU library's Python binding (loads libmoe.so; fails loudly if absent)."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    import token_routing_expert_router_amd as moe
    moe.load()
    return moe
