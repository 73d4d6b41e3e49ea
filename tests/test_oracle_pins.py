"""CPU: the fp64 oracle against library, brute-force, closed-form, golden and
invariant pins (see tests/oracle_pins.py for what each pin fixes)."""

import pytest

from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin()
