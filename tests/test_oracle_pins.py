"""The oracle checked against its pins (CPU only)."""
import pytest

import oracle
from tests import oracle_pins


@pytest.fixture(scope="module")
def lib():
    return oracle.load()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin, lib):
    pin(lib)


@pytest.mark.parametrize("fn", ["attention", "attention_rows"])
def test_mixed_input_dtypes_rejected(fn, lib):
    """q, k and v are read in one stored format: mixing them is an error,
    not a read of one array in another's element size."""
    import numpy as np
    q = np.zeros((1, 1, 4, 8))
    kv = np.zeros((1, 1, 4, 8), np.float32)
    call = getattr(oracle, fn)
    args = (q, q, kv, True, 0.5) + (([(0, 0, 1)],) if fn == "attention_rows" else ())
    with pytest.raises(TypeError):
        call(*args, lib=lib)
