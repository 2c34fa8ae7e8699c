"""The fp64 oracle against its pins (values printed on the pages, closed
forms, invariants, brute force, torch float64 CPU routines)."""
import pytest

from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_oracle_pin(pin):
    pin()
