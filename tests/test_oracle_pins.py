"""The oracle, pinned to the format definitions, the pages' byte figures,
independent library computations and invariants (CPU only)."""
import pytest

import oracle
import pins


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check(oracle.lib())
