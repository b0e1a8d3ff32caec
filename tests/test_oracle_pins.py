"""The CPU oracle against its pins (hand-worked examples, library routines,
closed forms and invariants of the MoE layer)."""
import pytest

import oracle
from tests import pins


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("check", pins.CHECKS, ids=lambda c: c.__name__)
def test_pin(orc, check):
    check(orc)
