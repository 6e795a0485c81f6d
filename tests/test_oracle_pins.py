"""The float64 oracle against closed forms, library special cases, brute force and the class table."""
import pytest

import oracle
from oracle_pins import ATTENTION_PINS, TOPK_PINS


@pytest.mark.parametrize("pin", ATTENTION_PINS + TOPK_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(oracle.load())
