"""The backward oracle against its pins (autograd of a separately written
recurrence, finite differences of the pinned forward oracle, a closed form,
packing invariance)."""
import pytest

import oracle
from oracle_bwd_pins import ALL_BWD_PINS


@pytest.mark.parametrize("pin", ALL_BWD_PINS, ids=[p.__name__ for p in ALL_BWD_PINS])
def test_bwd_pin(pin):
    pin(oracle.gdr_bwd, oracle.gdr_fwd)
