"""The CPU oracle against its pins (closed forms, invariants, exact arithmetic)."""
import pytest

import oracle
from oracle_pins import PINS


@pytest.fixture(scope="module")
def orc():
    return oracle.Oracle()


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(orc, pin):
    pin(orc)


def test_rejects_bad_shapes(orc):
    import numpy as np
    x = np.zeros((2, 12), dtype=np.uint16)
    c = np.ones((4, 4), dtype=np.float32)
    with pytest.raises(ValueError):  # hidden != heads * head_dim
        orc.rmsnorm_rope(x, None, c, c, heads=2, head_dim=8)
    c = np.ones((4, 2), dtype=np.float32)
    with pytest.raises(ValueError):  # odd head_dim
        orc.rmsnorm_rope(np.zeros((2, 10), dtype=np.uint16), None, c, c, heads=2, head_dim=5)
