"""The MXFP4 weight oracle against its pins (CPU only)."""
import pytest

from tests import pins


@pytest.mark.parametrize("pin", pins.QUANT_PINS, ids=lambda f: f.__name__)
def test_quant_pin(pin):
    pin()
