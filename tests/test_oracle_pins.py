"""CPU tests: the fp64 oracle against the facts the pages and the mathematics
fix (printed worked example, closed forms, brute force, invariants)."""
import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=[p.__name__ for p in pins.ALL_PINS])
def test_pin(orc, pin):
    pin(orc)
