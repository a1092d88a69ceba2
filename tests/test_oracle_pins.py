"""The oracle against what the pages and the mathematics fix (CPU only)."""
import pytest

import oracle_pins


@pytest.mark.parametrize("check", oracle_pins.CHECKS, ids=lambda f: f.__name__[len("check_"):])
def test_pin(O, check):
    check(O)
