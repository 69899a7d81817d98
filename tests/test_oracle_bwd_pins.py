"""The backward oracle against its pins (CPU only)."""
import pytest

from oracle_bwd_pins import ALL_BWD_PINS


@pytest.mark.parametrize("pin", ALL_BWD_PINS, ids=lambda f: f.__name__)
def test_bwd_pin(pin):
    pin()
