"""Checks that pin the fp64 packed-batch / sliding-window oracle to facts other
than itself.

Each ``pin_*`` takes ``vref(q, k, v, cu_seqlens, causal, scale, left, right)``
(q bf16 bits [H_q, total, D], k, v [H_kv, total, D]) -> (o, lse) and raises
AssertionError when a result contradicts the (separately pinned) forward
oracle, torch's SDPA with an explicit mask, a closed form or the locality of
the window.  They run on the real oracle (test_oracle_varlen_pins.py) and on
copies with planted mistakes (test_oracle_varlen_mutations.py).

What is pinned: attention within each sequence of a packed batch (variable
sequence lengths, page "AVO算法优化Transformer注意力机制性能解析", section 6) with
the local-window / band rule i-left <= j <= i+right (page "注意力机制的本质与计算
挑战", section 2.1), over the forward's definition.
"""
from __future__ import annotations

import numpy as np
import scipy.special
import torch

import oracle
from tests.oracle_pins import SCALE, bits_to64, close, rnd


def _fwd(q, k, v, causal):
    """Forward oracle on one sequence given as [H, n, D] arrays."""
    o, l = oracle.attn_ref(q[None], k[None], v[None], causal, SCALE, n_threads=1)
    return o[0], l[0]


def _packed(seed, Hq, Hkv, lens, D=16):
    total = int(sum(lens))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return (rnd(seed, (Hq, total, D)), rnd(seed + 1, (Hkv, total, D)),
            rnd(seed + 2, (Hkv, total, D)), cu)


def pin_varlen_sequences_are_independent(vref):
    """Each sequence of a packed batch (lengths 0, 1, 7, 33, 64) equals the
    forward oracle run on that sequence alone, in both mask modes."""
    q, k, v, cu = _packed(1500, 4, 2, [7, 1, 33, 0, 64])
    for causal in (False, True):
        o, lse = vref(q, k, v, cu, causal, SCALE, -1, -1)
        for s in range(len(cu) - 1):
            a, b = cu[s], cu[s + 1]
            if b == a:
                continue
            fo, fl = _fwd(q[:, a:b], k[:, a:b], v[:, a:b], causal)
            close(o[:, a:b], fo, tol=1e-13, what=f"sequence {s} O causal={causal}")
            close(lse[:, a:b], fl, tol=1e-13, what=f"sequence {s} LSE causal={causal}")


def _band(n, left, right, causal):
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    ok = np.ones((n, n), bool)
    if left >= 0:
        ok &= j >= i - left
    if right >= 0:
        ok &= j <= i + right
    if causal:
        ok &= j <= i
    return ok


def pin_window_library(vref):
    """Band masks against torch's fp64 SDPA with the explicit boolean mask and
    scipy's logsumexp of the masked scores (one sequence, GQA)."""
    q, k, v, cu = _packed(1600, 4, 2, [45])
    g = 2
    qt = torch.from_numpy(bits_to64(q))
    kt = torch.from_numpy(bits_to64(k)).repeat_interleave(g, dim=0)
    vt = torch.from_numpy(bits_to64(v)).repeat_interleave(g, dim=0)
    for left, right, causal in ((5, 5, False), (0, 3, False), (7, -1, True), (-1, 2, False),
                                (12, 0, True), (0, 0, False)):
        o, lse = vref(q, k, v, cu, causal, SCALE, left, right)
        ok = torch.from_numpy(_band(45, left, right, causal))
        eo = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=ok,
                                                              scale=SCALE).numpy()
        s = SCALE * np.matmul(qt.numpy(), np.swapaxes(kt.numpy(), -1, -2))
        s = np.where(ok.numpy(), s, -np.inf)
        what = f"window ({left}, {right}) causal={causal}"
        close(o, eo, tol=1e-12, what=what)
        close(lse, scipy.special.logsumexp(s, axis=-1), tol=1e-12, what=what + " LSE")


def pin_window_closed_forms(vref):
    """Window 0 on both sides (or left 0 with causal): each row sees only itself,
    O = V[i] exactly and LSE = scale * q_i.k_i.  Windows wider than the sequence
    change nothing (bitwise)."""
    q, k, v, cu = _packed(1700, 2, 2, [9, 20])
    qf, kf, vf = bits_to64(q), bits_to64(k), bits_to64(v)
    for left, right, causal in ((0, 0, False), (0, 5, True)):
        o, lse = vref(q, k, v, cu, causal, SCALE, left, right)
        assert np.array_equal(o, vf), f"window ({left}, {right}): O != V[i]"
        close(lse, SCALE * np.sum(qf * kf, axis=-1), what="self-only LSE")
    for causal in (False, True):
        a = vref(q, k, v, cu, causal, SCALE, -1, -1)
        b = vref(q, k, v, cu, causal, SCALE, 25, 30)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]), "wide window"


def pin_window_locality(vref):
    """Changing keys and values outside row i's window leaves row i unchanged
    (bitwise), and changing one inside it does not."""
    q, k, v, cu = _packed(1800, 2, 1, [40])
    i, left, right = 20, 4, 6
    k2, v2 = k.copy(), v.copy()
    outside = [j for j in range(40) if j < i - left or j > i + right]
    k2[:, outside] = rnd(1810, k2[:, outside].shape, 3.0)
    v2[:, outside] = rnd(1811, v2[:, outside].shape)
    a = vref(q, k, v, cu, False, SCALE, left, right)
    b = vref(q, k2, v2, cu, False, SCALE, left, right)
    assert np.array_equal(a[0][:, i], b[0][:, i]) and np.array_equal(a[1][:, i], b[1][:, i])
    k3 = k.copy()
    k3[:, i + right] = rnd(1812, k3[:, i + right].shape, 3.0)
    c = vref(q, k3, v, cu, False, SCALE, left, right)
    assert not np.array_equal(a[1][:, i], c[1][:, i]), "a key inside the window was ignored"


def pin_varlen_nonfinite(vref):
    """Non-finite values stay in their sequence and window: a NaN in V at the
    first token of sequence 1 makes that element NaN in exactly the rows of
    sequence 1 that see it (window and causal rule), and leaves every other
    element bitwise unchanged; a row of sequence 2 whose scores are all -inf is
    NaN (O and LSE)."""
    Hq, Hkv, lens = 2, 1, [5, 7, 6]
    q, k, v, cu = _packed(4100, Hq, Hkv, lens)
    s1 = int(cu[1])
    v2 = v.copy()
    v2[0, s1, 3] = 0x7FC0
    q3, k3 = q.copy(), k.copy()
    s2 = int(cu[2])
    k3[0, s2:, 9] = 0xBF80          # -1 in dim 9 for every key of sequence 2
    q3[1, s2 + 2, 9] = 0x7F80       # +inf: every score of that row is -inf
    for causal in (False, True):
        for left, right in ((-1, -1), (2, 0), (1, 3)):
            o0, l0 = vref(q, k, v, cu, causal, SCALE, left, right)
            o2, l2 = vref(q, k, v2, cu, causal, SCALE, left, right)
            hit = np.zeros(o0.shape, bool)
            for i in range(s1, s2):
                lo = max(s1, i - left) if left >= 0 else s1
                hi = min(s2 - 1, i + right) if right >= 0 else s2 - 1
                if causal:
                    hi = min(hi, i)
                if lo <= s1 <= hi:
                    hit[:, i, 3] = True
            assert np.all(np.isnan(o2[hit])), "NaN must reach the rows that see its key"
            assert np.array_equal(o2[~hit], o0[~hit]) and np.array_equal(l2, l0), "NaN spread"
            o3, l3 = vref(q3, k3, v, cu, causal, SCALE, left, right)
            assert np.all(np.isnan(o3[1, s2 + 2])) and np.isnan(l3[1, s2 + 2]), "all -inf row"


ALL_PINS = [pin_varlen_nonfinite, pin_varlen_sequences_are_independent, pin_window_library, pin_window_closed_forms,
            pin_window_locality]
