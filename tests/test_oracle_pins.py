"""The CPU oracle against its pins (no GPU needed)."""
import pytest

import oracle
from tests import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle)
