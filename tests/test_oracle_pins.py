"""The fp64 oracle against what the pages print, closed forms, library routines and
brute-force guarantees (CPU only)."""
import pytest

import oracle_pins
from oracle import oracle as oracle_mod


@pytest.fixture(scope="module")
def O():
    return oracle_mod.default()


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(O, check):
    check(O)
