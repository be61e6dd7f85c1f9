"""The fp64 backward oracle against finite differences of the forward oracle,
torch's fp64 autograd, hand-derived values, closed forms and invariants
(CPU only)."""
import numpy as np
import pytest

import oracle
import synth
from tests import oracle_bwd_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle.attn_bwd_ref)


def test_thread_count_does_not_change_result():
    w = synth.WORKLOADS["mha_tiny_b1_h2_n256"]
    q, k, v = w.generate()
    do = synth.normal_bf16(99, q.shape)
    a = oracle.attn_bwd_ref(q, k, v, do, True, w.scale, n_threads=1)
    b = oracle.attn_bwd_ref(q, k, v, do, True, w.scale, n_threads=7)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_bad_arguments_rejected():
    q = np.zeros((1, 3, 4, 8), np.uint16)
    k = np.zeros((1, 2, 4, 8), np.uint16)
    with pytest.raises(ValueError):
        oracle.attn_bwd_ref(q, k, k, q, False, 1.0)          # 3 % 2 != 0
    q2 = np.zeros((1, 2, 4, 8), np.uint16)
    with pytest.raises(ValueError):
        oracle.attn_bwd_ref(q2, k, k, q2, False, 1.0, rows=np.array([8]))
    with pytest.raises(ValueError):
        oracle.attn_bwd_ref(q2, k, k, q, False, 1.0)         # dO shape
