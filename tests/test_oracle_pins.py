"""The CPU oracle against what the pages and mathematics fix (no GPU)."""
import pytest

import oracle_pins as P


@pytest.mark.parametrize("pin", P.PINS, ids=[p.__name__ for p in P.PINS])
def test_pin(pin):
    pin()


def test_skewed_workloads():
    P.pin_skewed_workloads()
