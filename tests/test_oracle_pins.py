"""The CPU oracle against closed forms, invariants, library routines and scalar brute force."""
import pytest

import pins


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_pin(check):
    check()
