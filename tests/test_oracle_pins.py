"""The CPU oracle against closed forms, torch's SDPA, brute force, invariants and
the pages' printed KV sizes (CPU only)."""
import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(oracle)
