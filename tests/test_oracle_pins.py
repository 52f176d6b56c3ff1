"""The oracle against brute force, hand-worked golden values, torch's dense
conv2d / autograd through the dense reconstruction, closed forms and the
adjoint identity.  CPU only."""
import pytest

from oracle import oracle as O
from tests import pins


@pytest.fixture(scope="module")
def orc():
    O.build(force=False)
    return O.default()


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)
