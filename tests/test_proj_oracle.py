"""The projection / conv-front oracle against its pins (CPU only)."""
import pytest

from oracle import proj
from tests import proj_pins as P


@pytest.mark.parametrize("name", sorted(P.ALL_CHECKS))
def test_proj_oracle_pin(name):
    P.ALL_CHECKS[name](proj)
