"""The float64 oracle against its pins (closed forms, golden values, library routines, brute force)."""

import pytest

import oracle_pins


@pytest.mark.parametrize("name", sorted(oracle_pins.ALL_PINS))
def test_pin(name):
    oracle_pins.ALL_PINS[name]()
