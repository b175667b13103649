"""The oracle against hand-derived values, a library routine and invariances."""
import pytest

import oracle.paged_ref as ref
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(pin):
    pin(ref)
