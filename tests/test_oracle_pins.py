"""The CPU oracle against closed forms, identities, torch's SDPA and finite differences."""
import pytest

from oracle import attention as oracle_attention

from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle_attention)
