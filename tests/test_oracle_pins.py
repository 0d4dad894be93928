"""The oracle against its pins (CPU only)."""
import pytest

import oracle
from tests import oracle_pins


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_closed_form_of_harmonic_number():
    """The closed form used by the harmonic pin, checked against the correctly
    rounded sum of the exact fp64 terms 1/k (truncation error ~ 1/(120 n^4))."""
    import math
    for n in (1000, 100_000, 1_000_000):
        exact = math.fsum(1.0 / k for k in range(1, n + 1))
        assert abs(oracle_pins.harmonic_closed_form(n) - exact) <= 1e-12 * exact


def test_tolerance_rule():
    import numpy as np
    S = np.array([10.0, np.nan, np.inf, 0.0, -np.inf])
    A = np.array([1e5, 1.0, np.inf, 0.0, np.inf])
    got = np.array([10.0 + 1.0000009, np.nan, np.inf, 1e-6, np.inf])
    ok = oracle.within_tolerance(got, S, A)
    assert ok.tolist() == [True, True, True, True, False]
    assert not oracle.within_tolerance([11.2], [10.0], [1e5])[0]
    assert not oracle.within_tolerance([np.nan], [1.0], [1.0])[0]
