import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(autouse=True)
def _close_instant_handles():
    """Every library handle a test opened is closed when the test ends (after the device has
    drained), so no handle outlives its test and none is left to the interpreter's exit."""
    yield
    mod = sys.modules.get("rank_compressed_backprop_amd")
    if mod is None:
        return
    torch = sys.modules.get("torch")
    if torch is not None and torch.cuda.is_available() and torch.cuda.is_initialized():
        torch.cuda.synchronize()
    mod.close_all()
