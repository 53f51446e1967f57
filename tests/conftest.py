import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(params=["tiled", "split", "split8"])
def fwd_kernel(request, monkeypatch):
    """Run a forward test once on each forward kernel: the tiled kernel (one
    workgroup per 128-row query tile) and the split-key kernel (one per 32-row
    block, the keys shared out over its four or, at d <= 64, eight waves).
    Without the override the library picks the split-key kernel only for grids
    smaller than the GPU."""
    monkeypatch.setenv("FA_FWD_SPLIT", {"tiled": "0", "split": "1", "split8": "8"}[request.param])
    return request.param
