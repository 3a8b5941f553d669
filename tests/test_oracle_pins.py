"""The CPU oracle against its pins (closed forms, invariants, brute force)."""

import pytest

import oracle.attention as oracle_impl
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(oracle_impl)
