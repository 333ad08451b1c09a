"""The oracle against closed forms, special cases, invariants and brute force (CPU)."""
import pytest

from tests import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()
