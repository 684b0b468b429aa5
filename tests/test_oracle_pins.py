"""The oracle against closed forms, invariants, special cases and brute
force (CPU only)."""

import pytest

from tests import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=[f.__name__ for f in P.ALL_PINS])
def test_pin(pin):
    pin()
