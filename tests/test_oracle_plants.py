"""Every planted mistake in the oracle must be caught by at least one pin.

Each plant is a one-line error built into a separate copy of the oracle on the
CPU (a tie broken the wrong way, a dropped exp, a capacity off by one, a
reversed order inside an expert, SiLU on the wrong operand, a transposed down
projection, one slot's weight used for all, the shared expert dropped). The
pins that pass on the real oracle must reject each of these copies.
"""
import pytest

import oracle
from tests import pins


@pytest.mark.parametrize("plant", oracle.PLANTS)
def test_plant_is_caught(plant):
    orc = oracle.Oracle(plant)
    caught = []
    for check in pins.CHECKS:
        try:
            check(orc)
        except AssertionError:
            caught.append(check.__name__)
    assert caught, f"planted mistake {plant} passed every pin"
