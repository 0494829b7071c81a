"""The oracle against its pins (CPU only)."""
import pytest

import oracle.reference as ref
import oracle.formats as fmt
from . import oracle_pins as pins


class _Both:
    """The reference module with the format helpers attached, as the checks expect."""
    def __getattr__(self, name):
        return getattr(ref, name) if hasattr(ref, name) else getattr(fmt, name)


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    check(_Both())
