"""The CPU oracle against its pins (closed forms, invariants, library routines
and the pages' full-recompute criterion).  CPU only."""
import pytest

import oracle_pins


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check()
