"""The CPU oracle against closed forms, printed numbers, invariants, library routines and
brute force (no GPU)."""
import pytest

import oracle.oracle as orc
from pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(orc)
