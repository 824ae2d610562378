"""The fp64 oracle against facts outside itself (CPU only)."""
import pytest

from tests import _pins


@pytest.mark.parametrize("check", _pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    assert check()
