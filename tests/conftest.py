import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session")
def gpu():
    """The GPU path's library, loaded; skips nothing: a GPU test without a
    GPU or without the built library fails loudly."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test collected on a machine without a GPU")
    from transformer_layer_amd import lib
    return lib.load()
