"""The CPU oracle against its pins (no GPU)."""
import pytest

import oracle_pins
from oracle import Oracle


@pytest.fixture(scope="module")
def orc():
    return Oracle()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)
