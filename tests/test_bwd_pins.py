"""Run the pins of the attention-backward oracle (tests/bwd_pins.py) against
the oracle library."""
import pytest

import oracle
from bwd_pins import BPINS


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("pin", BPINS, ids=[p.__name__ for p in BPINS])
def test_bwd_pin(orc, pin):
    pin(orc)
