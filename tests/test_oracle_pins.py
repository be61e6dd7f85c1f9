"""The fp64 oracle against closed forms, invariants, library routines and the
pages' printed numbers (CPU only)."""
import json
import os

import numpy as np
import pytest

import oracle
import synth
from tests import oracle_pins as P

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle.attn_ref)


def test_score_count_printed_on_page():
    """The page prints the size of one N=4096 score matrix; the workload's pair
    count (which the throughput metric is built on) must reproduce it."""
    with open(os.path.join(GOLDEN, "score_count_n4096.json")) as f:
        g = json.load(f)
    w = synth.Workload("count", 1, 1, 1, g["n"])
    assert w.pairs == g["elements"]
    assert w.flops == 4 * 128 * g["elements"]


def test_thread_count_does_not_change_result():
    w = synth.WORKLOADS["mha_tiny_b1_h2_n256"]
    q, k, v = w.generate()
    o1, l1 = oracle.attn_ref(q, k, v, True, w.scale, n_threads=1)
    o7, l7 = oracle.attn_ref(q, k, v, True, w.scale, n_threads=7)
    assert np.array_equal(o1, o7) and np.array_equal(l1, l7)


def test_bad_arguments_rejected():
    q = np.zeros((1, 3, 4, 8), np.uint16)
    k = np.zeros((1, 2, 4, 8), np.uint16)
    with pytest.raises(ValueError):
        oracle.attn_ref(q, k, k, False, 1.0)          # 3 % 2 != 0
    with pytest.raises(ValueError):
        oracle.attn_ref(q[:, :2], k, k, False, 1.0, rows=[8])  # row out of range
