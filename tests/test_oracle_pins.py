"""The oracle against brute force, library routines, closed forms and the pages' invariants."""
import pytest

from tests import oracle_pins


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check()
