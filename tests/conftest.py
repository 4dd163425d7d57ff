import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


import pytest  # noqa: E402


@pytest.fixture
def plan():
    """Set launch-plan knobs of the HIP library for one test
    (``plan("pass2_generic", 1)``); every knob is back at its default after
    the test, whatever its outcome."""
    import gated_bidirectional_linear_amd as gla

    def set_knob(name, value):
        gla.plan_override(name, int(value))

    yield set_knob
    gla.plan_reset()
