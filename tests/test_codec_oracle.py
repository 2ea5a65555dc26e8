"""The int8 block codec oracle against its pins (CPU only)."""
import pytest

from oracle import codec
from tests import codec_pins as P


@pytest.mark.parametrize("name", sorted(P.ALL_CHECKS))
def test_codec_oracle_pin(name):
    P.ALL_CHECKS[name](codec)


def test_num_blocks():
    assert [codec.num_blocks(n, 128) for n in (1, 127, 128, 129, 256, 257)] == [1, 1, 1, 2, 2, 3]
