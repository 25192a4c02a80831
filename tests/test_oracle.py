"""CPU oracle against its pins (no GPU)."""
import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_oracle_pin(pin):
    pin(oracle.default())


def test_oracle_rejects_bad_points():
    import numpy as np
    a = np.zeros(4, np.uint16)
    with pytest.raises(ValueError):
        oracle.gemm_epi_points(2, 2, 1, 1, a, a, points=[(0, 2, 0)], ab="f16")
