import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs through the C-ABI library")
    config.addinivalue_line("markers", "slow: large oracle work (seconds to a minute on the CPU)")


def gpu_available():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def lib():
    """The loaded C-ABI library (built in-tree); fails loudly if it is missing."""
    import rollout_rlk_linear_amd as rlk
    return rlk.load_library()
