"""The CPU oracle against what the definition fixes independently of it."""
import pytest

import _oracle_pins as pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin()
