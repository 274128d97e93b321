"""The oracle against its pins (CPU only).

Each pin ties the float64 oracle to something outside itself: a hand-derived
closed form (golden/rational_case.json), invariants of the softmax, a
pure-Python brute force, torch float64 routines, finite differences and
gradient identities.  See pins.py for what each one checks.
"""

import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    failures = pin()
    assert not failures, "\n".join(failures)
