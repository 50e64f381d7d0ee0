"""The CPU oracle against its pins (closed forms, library routines, hand-worked
examples, brute force and the invariants the pages state). CPU only."""
import pytest

import oracle
import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle.kpool_oracle)
