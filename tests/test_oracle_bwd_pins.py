"""The backward oracle against its pins (CPU only)."""

import pytest

import oracle
import oracle_bwd_pins


@pytest.mark.parametrize("pin", oracle_bwd_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_backward_oracle_pin(pin):
    pin(oracle.attention_bwd)
