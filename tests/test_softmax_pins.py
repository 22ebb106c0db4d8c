"""The row-softmax oracle against its pins (see tests/softmax_pins.py)."""
import pytest

import oracle
from tests import softmax_pins as pins


@pytest.mark.parametrize("pin", pins.SOFTMAX_PINS, ids=lambda f: f.__name__)
def test_softmax_pin(pin):
    pin(oracle.softmax_rows)
