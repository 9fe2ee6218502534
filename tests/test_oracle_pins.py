"""The CPU oracle against its pins (no GPU)."""
import os, sys
sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

import pytest

import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin()
