"""The CPU oracle against codecs, closed forms, exact arithmetic and invariants."""

import pytest

import oracle_pins as pins


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check()
