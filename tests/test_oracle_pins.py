"""The fp64 oracle against the pages' worked examples, hand-derived values,
torch's float64 SDPA, closed forms, invariants and brute force (CPU only)."""

import pytest

import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()
