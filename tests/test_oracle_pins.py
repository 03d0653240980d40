"""The oracle against its pins (page values, closed forms, library routines,
invariants, brute force).  CPU only."""
import pytest

import oracle.oracle as O
import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(O)
