import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


import pytest


@pytest.fixture
def force_plan():
    """Test-only plan overrides (aq_debug_force_plan): force_plan("PREFILL_BM", 256)
    forces one knob on this thread; every knob is reset when the test ends."""
    from rank_shared_block_amd import binding as B

    def set_knob(name, value):
        B.debug_force_plan(name, value)

    yield set_knob
    B.aq_debug_reset_plan()
