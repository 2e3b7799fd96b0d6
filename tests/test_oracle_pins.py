"""The fp64 oracle against its pins (closed forms, invariants, SDPA, brute force)."""
import pytest

import oracle.reference as O
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(O)
