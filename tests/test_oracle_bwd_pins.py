"""The backward oracle against finite differences, library autograd and invariants (CPU only)."""

import pytest

from . import oracle_bwd_pins

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


@pytest.mark.parametrize("pin", oracle_bwd_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()
