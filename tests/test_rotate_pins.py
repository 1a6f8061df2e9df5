"""Run the pins of the incoherent-processing oracle (tests/rotate_pins.py)
against the oracle library."""
import pytest

import oracle
from rotate_pins import RPINS


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("pin", RPINS, ids=[p.__name__ for p in RPINS])
def test_rotate_pin(orc, pin):
    pin(orc)
