"""The CPU oracle against its pins (runs without a GPU)."""
import pytest

import oracle
from tests import oracle_pins


@pytest.fixture(scope="module")
def orc():
    return oracle.load()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_threads(orc):
    assert orc.set_threads(0) >= 1
