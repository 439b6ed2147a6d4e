"""The fp64 oracle against library routines, closed forms and the pages' invariants (CPU)."""
import pytest

import oracle.attention as orc
from oracle_checks import ALL_CHECKS


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check(orc)
