"""The fp64 FP8 (e4m3) oracle against torch's float8_e4m3fn, the format's own
values, the bf16-input forward oracle, torch SDPA and closed forms (CPU only)."""
import numpy as np
import pytest

import oracle
from tests import oracle_fp8_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle.attn_fp8_ref, oracle.e4m3_decode)


def test_bad_arguments_rejected():
    q = np.zeros((1, 3, 4, 8), np.uint8)
    k = np.zeros((1, 2, 4, 8), np.uint8)
    with pytest.raises(ValueError):
        oracle.attn_fp8_ref(q, k, k, 1.0, 1.0, 1.0, False, 1.0)          # 3 % 2 != 0
    with pytest.raises(ValueError):
        oracle.attn_fp8_ref(q[:, :2], k, k, 1.0, 1.0, 1.0, False, 1.0, rows=[8])   # row out of range
