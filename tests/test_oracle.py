"""The CPU oracle against closed forms, invariants, scipy and finite differences."""
import pytest

import oracle.attention as ora
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(ora)
