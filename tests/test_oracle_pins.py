"""The oracle against what the pages and the mathematics fix (CPU only)."""
import pytest

import oracle_pins


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda c: c.__name__[6:])
def test_oracle_pin(check, oracle_lib):
    check(oracle_lib)
