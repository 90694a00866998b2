"""The fp64 oracle against hand-worked values, library routines, the matrix form
of the recurrence, closed forms, invariants and the pages' examples."""
import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)
