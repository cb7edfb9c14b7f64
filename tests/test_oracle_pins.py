"""The oracle against its pins (CPU only)."""
import pytest

import oracle
from tests import oracle_pins


@pytest.fixture(scope="module")
def orc():
    oracle.build()
    return oracle.Oracle(oracle.LIBRARY)


@pytest.mark.parametrize("pin", oracle_pins.PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    assert orc.plant == 0
    pin(orc)
