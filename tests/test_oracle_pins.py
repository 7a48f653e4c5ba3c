"""The oracle against what the pages and the mathematics fix (CPU only)."""

import pytest

from oracle_pin_checks import ALL_CHECKS


@pytest.mark.parametrize("check", ALL_CHECKS, ids=[c.__name__ for c in ALL_CHECKS])
def test_pin(check):
    check()
