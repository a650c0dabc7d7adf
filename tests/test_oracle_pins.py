"""The fp64 reference against its pins (CPU only)."""
import pytest

import oracle
from oracle_pins import PINS


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(orc, pin):
    pin(orc)


def test_rejects_invalid_shapes(orc):
    import numpy as np
    q = np.zeros((4, 2))
    k = np.zeros((3, 2))
    with pytest.raises(ValueError):
        orc.attention(q, k, k, causal=True, scale=1.0)   # causal needs Nq <= Nkv
    with pytest.raises(ValueError):
        orc.attention(q, np.zeros((0, 2)), np.zeros((0, 2)), causal=False, scale=1.0)
