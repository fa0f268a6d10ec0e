"""The CPU oracle against facts fixed outside it (runs without a GPU)."""
import pytest

from tests import oracle_pins


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check, oracle_lib):
    check(oracle_lib)
