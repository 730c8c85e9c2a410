"""The expert-FFN oracle against its pins (CPU only)."""
import pytest

from tests import pins


@pytest.mark.parametrize("pin", pins.FFN_PINS, ids=lambda f: f.__name__)
def test_ffn_pin(pin):
    pin()
