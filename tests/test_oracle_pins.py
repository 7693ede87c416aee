"""The CPU oracle against its pins (closed forms, brute force, fixtures)."""
import pytest

from oracle_pins import PINS


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin, oracle_lib):
    pin(oracle_lib)
