"""The CPU oracle against its pins (closed forms, error bounds, brute force,
library routines on special cases, and the properties the pages state)."""
import pytest

import oracle_checks as oc


@pytest.mark.parametrize("check", oc.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(olib, check):
    check(olib)
