"""The attention-block oracle against loops, head permutations, linearity and padding (CPU only)."""

import pytest

from . import oracle_block_pins


@pytest.mark.parametrize("pin", oracle_block_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()
