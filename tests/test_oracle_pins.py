"""The oracle against the pages' printed values, closed forms, a library
attention on contiguous keys, element-wise brute force, and invariants."""

import pytest

import oracle_pins as pins


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    check()
