"""CPU-only pins of the float64 oracle (see tests/oracle_checks.py)."""
import pytest

import oracle
from tests import oracle_checks as chk


@pytest.mark.parametrize("check", chk.ALL, ids=[c.__name__ for c in chk.ALL])
def test_oracle_pin(check):
    check(oracle)
