"""The oracle against its pins (CPU only)."""
import pytest

import oracle_pins as pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin, olib):
    pin(olib)
