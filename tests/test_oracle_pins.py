"""The CPU oracle against the pins (worked example, closed forms, invariants, library routines)."""
import pytest

import oracle
import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle.dsv4_oracle)
