import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


import pytest  # noqa: E402


@pytest.fixture
def knobs():
    """Set library knobs (lattn_set_knob) inside a test; every knob touched is restored
    to its previous value when the test ends."""
    from decayed_recurrent_attention_amd import lattn

    touched = {}

    def setter(which, value):
        prev = lattn.lattn_set_knob(which, value)
        touched.setdefault(which, prev)

    yield setter
    for which, prev in touched.items():
        lattn.lattn_set_knob(which, prev)
