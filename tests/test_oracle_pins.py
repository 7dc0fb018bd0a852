"""The oracle against what the pages and mathematics fix (CPU only)."""
import pytest

import oracle_pins as pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(O, pin):
    pin(O)
