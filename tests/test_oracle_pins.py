"""The CPU oracle against its pins (no GPU)."""
import pytest

from oracle import oracle as oracle_mod
from tests import oracle_pins


@pytest.fixture(scope="module")
def orc():
    return oracle_mod.default()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


@pytest.mark.parametrize("pin", oracle_pins.APPEND_PINS, ids=lambda f: f.__name__)
def test_append_pin(orc, pin):
    pin(orc)


@pytest.mark.parametrize("pin", oracle_pins.MULTI_PINS, ids=lambda f: f.__name__)
def test_multi_pin(orc, pin):
    pin(orc)


def test_rejects_bad_arguments(orc):
    import numpy as np
    q = np.zeros((1, 3, 4))
    k = np.zeros((1, 2, 5, 4))
    with pytest.raises(ValueError):
        orc.decode(q, k, k, 1.0)           # Hq not a multiple of Hkv
    q = np.zeros((1, 2, 4))
    with pytest.raises(ValueError):
        orc.decode(q, k, k, 1.0, seq_lens=np.array([6], np.int32))  # length > T
    with pytest.raises(ValueError):
        orc.decode(q, k, k, 1.0, rows=[2])  # row out of range
