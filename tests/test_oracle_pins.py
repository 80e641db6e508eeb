"""The float64 oracle against facts that do not come from it (CPU only)."""
import pytest

from oracle import build_oracle
from tests.oracle_pins import ALL_CHECKS


@pytest.fixture(scope="module")
def lib():
    return build_oracle()


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_pin(lib, check):
    check(lib)
