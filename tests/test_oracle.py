"""The CPU oracle against its pins (see tests/oracle_pins.py)."""
import pytest

import oracle
import oracle_pins as pins


@pytest.fixture(scope="module")
def lib():
    return oracle.load()


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(lib, pin):
    pin(lib)
