"""The CPU oracle against its pins (hand-derived values, closed forms, exact
arithmetic, library special cases, exhaustive search).  No GPU needed."""
import pytest

import pins


@pytest.mark.parametrize("check", pins.ALL, ids=[c.__name__ for c in pins.ALL])
def test_pin(check):
    check()
