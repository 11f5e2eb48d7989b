"""The fp64 oracle against its pins (closed forms, brute force, a library
routine and invariances); see tests/pins.py for the sources of each."""
import pytest

import oracle
from pins import PINS


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(oracle)
