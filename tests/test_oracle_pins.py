"""The oracle against its pins (closed forms, exact arithmetic, an independent
chunked derivation, invariants and the pages' printed magnitudes)."""
import pytest

import oracle
from oracle_pins import ALL_PINS, pin_page_magnitudes


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(pin):
    pin(oracle.gdr_fwd)


def test_page_magnitudes_long():
    """The T = 20468 row of the printed max_ref table."""
    pin_page_magnitudes(oracle.gdr_fwd, T=20468)


def test_thread_count_is_reported():
    assert oracle.threads_used(3, 100) == 3
    assert oracle.threads_used(8, 2) == 2
    assert oracle.threads_used(0, 10 ** 6) >= 1
