"""The CPU oracle against its pins (closed forms, hand-written golden masks,
library routines, invariants).  CPU only."""
import pytest

import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=[f.__name__ for f in P.ALL_PINS])
def test_pin(pin, oracle_lib):
    pin(oracle_lib)
