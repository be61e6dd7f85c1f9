"""The fp64 block-sparse oracle against the dense and packed-batch oracles,
torch SDPA with the expanded mask, closed forms and mask locality (CPU only)."""
import numpy as np
import pytest

import oracle
from synth import lists_to_csr
from tests import oracle_blocksparse_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle.attn_blocksparse_ref)


def test_bad_arguments_rejected():
    q = np.zeros((1, 2, 16, 8), np.uint16)
    ptr, idx = lists_to_csr([[0], [1]])
    with pytest.raises(ValueError):
        oracle.attn_blocksparse_ref(q, q, q, ptr[:2], idx, 8, False, 1.0)      # too few offsets
    with pytest.raises(ValueError):
        oracle.attn_blocksparse_ref(q, q, q, np.array([0, 2, 1], np.int32), idx, 8, False, 1.0)
    with pytest.raises(ValueError):   # three mask heads for two query heads
        oracle.attn_blocksparse_ref(q, q, q, *lists_to_csr([[0], [1]] * 3), 8, False, 1.0)
