"""The oracle against facts fixed outside it (CPU only).

Each pin lives in ``oracle_pins.py``; see that module for what each checks.
"""
import pytest

import oracle
from oracle_pins import PINS


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(orc, pin):
    pin(orc)
