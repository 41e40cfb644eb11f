"""The oracle against what the pages and the mathematics fix (CPU only)."""

import pytest

from . import oracle_pins

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()
