"""The oracle against its pins (CPU only)."""
import pytest

import oracle
import oracle_checks


@pytest.fixture(scope="module")
def orc():
    return oracle.Oracle()


@pytest.mark.parametrize("check", oracle_checks.ALL_CHECKS,
                         ids=[c.__name__ for c in oracle_checks.ALL_CHECKS])
def test_oracle_pin(orc, check):
    check(orc)
