"""Pins of the CPU oracle (P1-P9 plus the statistics), run on the CPU."""
import pytest

import oracle as O
from pins import ALL_CHECKS


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check(O)
