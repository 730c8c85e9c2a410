"""The routing oracle against its pins (CPU only)."""
import pytest

from tests import pins


@pytest.mark.parametrize("pin", pins.ROUTING_PINS, ids=lambda f: f.__name__)
def test_routing_pin(pin):
    pin()


def test_lexsort_pin_sees_ties():
    # bf16 spacing makes ties common at E=128; the pin must actually exercise them
    assert pins.pin_topk_lexsort() > 50


@pytest.mark.parametrize("e,k", [(32, 4), (128, 4), (64, 8), (8, 2), (5, 5), (1, 1)])
def test_invariants_shapes(e, k):
    pins.pin_metadata_invariants(n=257, e=e, k=k, seed=e * 31 + k)
