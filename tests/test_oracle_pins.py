"""The CPU oracle against its pins (closed forms, brute force, invariants,
library routines of another algorithm, finite differences)."""
import pytest

from tests import pins

CHECKS = [name for name in dir(pins) if name.startswith("check_")]


@pytest.mark.parametrize("name", CHECKS)
def test_pin(name):
    getattr(pins, name)()
