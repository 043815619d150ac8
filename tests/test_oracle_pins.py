"""The oracle against its pins (CPU only)."""
import pytest

import oracle as O
from oracle_pins import PINS


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(O.load())
