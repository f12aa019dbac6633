"""The CPU oracle against its pins (hand-worked fixtures, brute force,
format definitions, torch's fp8 cast, invariants and closed forms)."""

import pytest

import oracle
import oracle_pins as pins


@pytest.fixture(scope="module")
def O():
    return oracle.default()


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(O, pin):
    pin(O)
