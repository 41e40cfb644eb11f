"""The BSHD document/padding oracle against THD packing, invariants and brute force (CPU only)."""

import pytest

from . import oracle_bshd_pins


@pytest.mark.parametrize("pin", oracle_bshd_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()
