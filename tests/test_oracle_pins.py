"""The CPU oracle against facts outside itself (hand-worked blocks, exact
rational arithmetic, integer arithmetic, invariants of the Q4_0 rule)."""

import pytest

import oracle_checks as oc
from oracle import q4_oracle


@pytest.mark.parametrize("check", oc.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check(q4_oracle)
