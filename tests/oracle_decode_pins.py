"""Checks that pin the fp64 decode and merge oracles to facts other than
themselves.

Each ``pin_*`` takes ``dref(q, k, v, causal, scale) -> (o, lse)`` and
``mref(o_part, lse_part) -> (o, lse)`` and raises AssertionError when a result
contradicts the (separately pinned) forward oracle, a library routine, a closed
form or an invariant.  They run on the real oracle (test_oracle_decode_pins.py)
and on copies with planted mistakes (test_oracle_decode_mutations.py).

What is pinned: M query rows that are the last M positions of a sequence whose
L keys and values are cached, with the forward's definition (page "GPU注意力算子
性能优化" (QiMeng-Attention), section 1), and the exact combination of partial
results over disjoint key sets (the QiMeng page, section 3.1.1: local
computation plus a global reduction).
"""
from __future__ import annotations

import numpy as np
import scipy.special
import torch

import oracle
from tests.oracle_pins import SCALE, bits_to64, close, rnd


def pin_decode_equals_forward_rows(dref, mref):
    """Decode rows are rows L-M..L-1 of the forward over L tokens (the other
    query rows of that forward are arbitrary): the causal forward's row L-M+i
    sees keys 0..L-M+i, the non-causal one all L keys."""
    for t, (B, Hq, Hkv, M, L, D) in enumerate(((1, 4, 2, 3, 29, 16), (2, 3, 1, 1, 40, 8),
                                               (1, 2, 2, 7, 7, 32))):
        qd = rnd(900 + t, (B, Hq, M, D))
        k, v = rnd(910 + t, (B, Hkv, L, D)), rnd(920 + t, (B, Hkv, L, D))
        qf = rnd(930 + t, (B, Hq, L, D))
        qf[:, :, L - M:] = qd
        for causal in (False, True):
            o, lse = dref(qd, k, v, causal, SCALE)
            of, lf = oracle.attn_ref(qf, k, v, causal, SCALE, n_threads=1)
            close(o, of[:, :, L - M:], tol=1e-13, what=f"decode vs forward rows causal={causal}")
            close(lse, lf[:, :, L - M:], tol=1e-13, what=f"decode LSE vs forward causal={causal}")


def pin_decode_library(dref, mref):
    """torch's fp64 CPU SDPA with an explicit bottom-right boolean mask, and
    scipy's logsumexp of the scaled scores."""
    for t, (B, Hq, Hkv, M, L, D) in enumerate(((1, 8, 2, 4, 33, 64), (1, 16, 1, 1, 100, 128),
                                               (2, 2, 2, 5, 5, 8), (1, 4, 4, 16, 70, 16))):
        q = rnd(950 + t, (B, Hq, M, D))
        k, v = rnd(960 + t, (B, Hkv, L, D)), rnd(970 + t, (B, Hkv, L, D))
        g = Hq // Hkv
        qt = torch.from_numpy(bits_to64(q))
        kt = torch.from_numpy(bits_to64(k)).repeat_interleave(g, dim=1)
        vt = torch.from_numpy(bits_to64(v)).repeat_interleave(g, dim=1)
        for causal in (False, True):
            o, lse = dref(q, k, v, causal, SCALE)
            allowed = np.ones((M, L), bool)
            if causal:
                allowed = np.arange(L)[None, :] <= (L - M + np.arange(M))[:, None]
            eo = torch.nn.functional.scaled_dot_product_attention(
                qt, kt, vt, attn_mask=torch.from_numpy(allowed), scale=SCALE).numpy()
            s = SCALE * np.matmul(qt.numpy(), np.swapaxes(kt.numpy(), -1, -2))
            s = np.where(allowed, s, -np.inf)
            close(o, eo, tol=1e-12, what=f"decode vs torch causal={causal}")
            close(lse, scipy.special.logsumexp(s, axis=-1), tol=1e-12,
                  what=f"decode LSE vs logsumexp causal={causal}")


def pin_decode_single_row(dref, mref):
    """M = 1: the one row is the last position, so the causal mask allows every
    key and both modes agree bitwise; L = 1 gives O = V[0], LSE = the one score."""
    q, k, v = rnd(980, (2, 4, 1, 32)), rnd(981, (2, 2, 60, 32)), rnd(982, (2, 2, 60, 32))
    a, la = dref(q, k, v, False, SCALE)
    b, lb = dref(q, k, v, True, SCALE)
    assert np.array_equal(a, b) and np.array_equal(la, lb), "M = 1 causal != non-causal"
    k1, v1 = k[:, :, :1], v[:, :, :1]
    o, lse = dref(q, k1, v1, True, SCALE)
    assert np.array_equal(o, np.repeat(bits_to64(v1), 2, axis=1)), "L = 1: O != V[0]"
    s = SCALE * np.sum(bits_to64(q) * np.repeat(bits_to64(k1), 2, axis=1), axis=-1)
    close(lse, s, what="L = 1 LSE")


def _split_partials(dref, q, k, v, bounds):
    """Partial (O, LSE) of non-causal decode over contiguous key ranges; an empty
    range is a part with LSE = -inf and O = 0."""
    B, Hq, M, D = q.shape
    ops, lps = [], []
    for lo, hi in bounds:
        if hi > lo:
            o, l = dref(q, k[:, :, lo:hi], v[:, :, lo:hi], False, SCALE)
        else:
            o, l = np.zeros((B, Hq, M, D)), np.full((B, Hq, M), -np.inf)
        ops.append(o.reshape(-1, D))
        lps.append(l.reshape(-1))
    return np.stack(ops, axis=1), np.stack(lps, axis=1)


def pin_merge_reassembles_split(dref, mref):
    """Merging the partial results of disjoint key ranges (one of them empty)
    gives the result over all keys, from the decode oracle."""
    B, Hq, Hkv, M, L, D = 1, 4, 2, 3, 57, 16
    q = rnd(990, (B, Hq, M, D))
    k, v = rnd(991, (B, Hkv, L, D)), rnd(992, (B, Hkv, L, D), 2.0)
    full_o, full_l = dref(q, k, v, False, SCALE)
    for bounds in (((0, 20), (20, 20), (20, 57)), ((0, 1), (1, 56), (56, 57)), ((0, 57),)):
        op, lp = _split_partials(dref, q, k, v, bounds)
        o, l = mref(op, lp)
        close(o, full_o.reshape(-1, D), tol=1e-12, what=f"merge of {bounds}")
        close(l, full_l.reshape(-1), tol=1e-12, what=f"merged LSE of {bounds}")


def pin_merge_closed_forms(dref, mref):
    """Equal LSEs a: LSE = a + ln P and O = mean of the parts; LSE agrees with
    numpy's logaddexp; a part 1000 nats above the others is returned unchanged
    (no overflow); a single part is the identity; all-empty rows give O = 0,
    LSE = -inf; a NaN LSE_p makes its row NaN, as numpy's logaddexp does, also
    when every other part is empty, and an empty part beside a finite one is
    left out."""
    rng = np.random.default_rng(7)
    op = rng.standard_normal((5, 3, 8))
    lp = np.full((5, 3), 1.5)
    o, l = mref(op, lp)
    close(o, op.mean(axis=1), what="equal-LSE mean")
    close(l, np.full(5, 1.5 + np.log(3.0)), what="equal-LSE LSE")
    lp2 = rng.standard_normal((5, 4)) * 3
    op2 = rng.standard_normal((5, 4, 8))
    _, l2 = mref(op2, lp2)
    close(l2, np.logaddexp.reduce(lp2, axis=1), what="logaddexp")
    lp3 = np.array([[1000.0, 0.0, -5.0]])
    op3 = rng.standard_normal((1, 3, 8))
    o3, l3 = mref(op3, lp3)
    close(o3, op3[:, 0], what="dominant part")
    close(l3, [1000.0], tol=1e-15, what="dominant LSE")
    o4, l4 = mref(op3[:, :1], lp3[:, :1])
    assert np.array_equal(o4, op3[:, 0]) and np.array_equal(l4, lp3[:, 0]), "single part"
    o5, l5 = mref(np.zeros((2, 2, 8)), np.full((2, 2), -np.inf))
    assert np.all(o5 == 0) and np.all(l5 == -np.inf), "all-empty row"
    lp6 = np.array([[np.nan, -np.inf], [0.5, np.nan], [-np.inf, 0.5]])
    op6 = rng.standard_normal((3, 2, 8))
    op6[2, 0] = 0.0
    o6, l6 = mref(op6, lp6)
    ref6 = np.logaddexp.reduce(lp6, axis=1)
    assert np.array_equal(np.isnan(l6), np.isnan(ref6)) and np.isnan(l6[:2]).all(), "NaN part LSE"
    assert np.isnan(o6[:2]).all() and np.isfinite(o6[2]).all(), "NaN part O"
    close(o6[2], op6[2, 1], what="empty part beside a finite one")
    close(l6[2:], [0.5], tol=1e-15, what="LSE beside an empty part")


def pin_merge_permutation(dref, mref):
    """Merging is independent of the order of the parts."""
    rng = np.random.default_rng(11)
    op = rng.standard_normal((6, 5, 16))
    lp = rng.standard_normal((6, 5)) * 4
    lp[2, 1] = -np.inf
    perm = rng.permutation(5)
    a, la = mref(op, lp)
    b, lb = mref(op[:, perm], lp[:, perm])
    close(b, a, tol=1e-14, what="permuted O")
    close(lb, la, tol=1e-14, what="permuted LSE")


ALL_PINS = [pin_decode_equals_forward_rows, pin_decode_library, pin_decode_single_row,
            pin_merge_reassembles_split, pin_merge_closed_forms, pin_merge_permutation]
