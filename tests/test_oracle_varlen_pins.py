"""The fp64 packed-batch / sliding-window oracle against the forward oracle,
torch SDPA with explicit masks, closed forms and window locality (CPU only)."""
import numpy as np
import pytest

import oracle
from tests import oracle_varlen_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle.attn_varlen_ref)


def test_bad_arguments_rejected():
    q = np.zeros((2, 10, 8), np.uint16)
    with pytest.raises(ValueError):
        oracle.attn_varlen_ref(q, q, q, np.array([0, 4, 9], np.int32), False, 1.0)   # total 10
    with pytest.raises(ValueError):
        oracle.attn_varlen_ref(q, q, q, np.array([0, 6, 4, 10], np.int32), False, 1.0)
