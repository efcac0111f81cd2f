"""The CPU oracle against its pins (hand-worked examples, library special
cases, brute force, closed forms, invariants). No GPU needed."""
import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(orc, pin):
    pin(orc)
