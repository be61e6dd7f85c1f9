"""The fp64 decode and merge oracles against the forward oracle, library
routines, closed forms and invariants (CPU only)."""
import numpy as np
import pytest

import oracle
from tests import oracle_decode_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle.attn_decode_ref, oracle.attn_lse_merge_ref)


def test_bad_arguments_rejected():
    q = np.zeros((1, 3, 2, 8), np.uint16)
    k = np.zeros((1, 2, 4, 8), np.uint16)
    with pytest.raises(ValueError):
        oracle.attn_decode_ref(q, k, k, False, 1.0)          # 3 % 2 != 0
    q2 = np.zeros((1, 2, 5, 8), np.uint16)
    with pytest.raises(ValueError):
        oracle.attn_decode_ref(q2, k, k, True, 1.0)          # causal needs M <= L
    with pytest.raises(ValueError):
        oracle.attn_lse_merge_ref(np.zeros((2, 3, 4)), np.zeros((2, 2)))
