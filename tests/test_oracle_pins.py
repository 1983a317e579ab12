"""The CPU oracle against its pins (no GPU)."""
import pytest

import oracle
from tests.oracle_pins import ALL_PINS


@pytest.fixture(scope="module")
def orc():
    oracle.build()
    return oracle.Oracle()


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(orc, pin):
    pin(orc)
