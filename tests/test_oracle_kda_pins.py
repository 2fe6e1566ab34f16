"""The per-channel-gate oracle against its pins (scalar reduction, the literal
matrix form, the chunk form, closed forms)."""
import pytest

import oracle
from oracle_kda_pins import ALL_KDA_PINS


@pytest.mark.parametrize("pin", ALL_KDA_PINS, ids=[p.__name__ for p in ALL_KDA_PINS])
def test_kda_pin(pin):
    pin(oracle.gdr_kda_fwd)
