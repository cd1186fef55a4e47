import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size parity case (minutes of CPU oracle work)")


@pytest.fixture(autouse=True)
def _automatic_slab_width(monkeypatch):
    # A caller's FLCE_SLAB_COLS would override the slab widths the tests choose
    # (they force them with FLCE_DEBUG_SLAB_COLS) and the sizes they expect.
    monkeypatch.delenv("FLCE_SLAB_COLS", raising=False)
