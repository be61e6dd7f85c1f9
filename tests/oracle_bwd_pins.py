"""Checks that pin the fp64 backward oracle to facts other than itself.

Each ``pin_*`` takes ``bref(q, k, v, do, causal, scale, rows=None, mags=False,
keys=None)``
(bf16 bit arrays in; float64 (dq, dk, dv) out, plus the error-scale sums when
``mags``) and raises AssertionError when the result contradicts finite
differences of the (separately pinned) forward oracle, a library autograd, a
hand-derived case, a closed form or an invariant of the gradient.  They run on
the real oracle (test_oracle_bwd_pins.py) and on copies with planted mistakes
(test_oracle_bwd_mutations.py), where at least one pin must fail for each.

What is pinned: the gradient of L = sum(dO * O) through the forward of page
"GPU注意力算子性能优化" (QiMeng-Attention), section 1, whose backward the AVO page
(section 2.2) and the QiMeng page (section 2.2.2) name without writing out.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle
from tests.oracle_pins import SCALE, bf, bits_to64, close, rnd


def _lsum(o, do):
    return float(np.sum(o * bits_to64(do)))


def _fwd(q, k, v, causal, scale):
    return oracle.attn_ref(q, k, v, causal, scale, n_threads=1)


def _grid(seed, shape, lo=-16, hi=17):
    """bf16-exact values on a 1/8 grid in [-2, 2]: x +- 1/16 stays exact."""
    g = np.random.default_rng(seed)
    return bf(g.integers(lo, hi, shape) / 8.0)


# -------------------------------------------------------- finite differences
def pin_bwd_finite_difference(bref):
    """Each gradient element vs a Richardson-extrapolated central difference of
    L = sum(dO * O), with O from the forward oracle.  Steps h = 1/32 and 1/16
    keep every perturbed input exact in bf16; the extrapolation's error is
    O(h^4)."""
    h = 1.0 / 32.0
    for (B, Hq, Hkv, N, D) in ((1, 2, 1, 6, 4), (1, 1, 1, 5, 3)):
        q, k, v = _grid(1, (B, Hq, N, D)), _grid(2, (B, Hkv, N, D)), _grid(3, (B, Hkv, N, D))
        do = rnd(4, (B, Hq, N, D))
        scale = 0.5
        for causal in (False, True):
            dq, dk, dv = bref(q, k, v, do, causal, scale)
            for name, arr, grad in (("dQ", q, dq), ("dK", k, dk), ("dV", v, dv)):
                x = bits_to64(arr)
                fd = np.empty_like(x)
                for idx in np.ndindex(*x.shape):
                    vals = []
                    for step in (h, -h, 2 * h, -2 * h):
                        xp = x.copy()
                        xp[idx] += step
                        args = {"dQ": (bf(xp), k, v), "dK": (q, bf(xp), v),
                                "dV": (q, k, bf(xp))}[name]
                        vals.append(_lsum(_fwd(*args, causal, scale)[0], do))
                    d1 = (vals[0] - vals[1]) / (2 * h)
                    d2 = (vals[2] - vals[3]) / (4 * h)
                    fd[idx] = (4 * d1 - d2) / 3
                close(grad, fd, tol=2e-6, what=f"FD {name} {B,Hq,Hkv,N,D} causal={causal}")


# ------------------------------------------------------------ library routine
def torch_grads_f64(q, k, v, do, causal, scale):
    """torch autograd through its fp64 CPU scaled_dot_product_attention, with
    K/V heads repeated per group (autograd sums the group's gradients)."""
    g = q.shape[1] // k.shape[1]
    qt = torch.from_numpy(bits_to64(q)).requires_grad_()
    kt = torch.from_numpy(bits_to64(k)).requires_grad_()
    vt = torch.from_numpy(bits_to64(v)).requires_grad_()
    o = torch.nn.functional.scaled_dot_product_attention(
        qt, kt.repeat_interleave(g, dim=1), vt.repeat_interleave(g, dim=1),
        is_causal=bool(causal), scale=float(scale))
    o.backward(torch.from_numpy(bits_to64(do)))
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


LIB_SHAPES = [(1, 1, 1, 1, 1), (1, 1, 1, 2, 2), (1, 2, 1, 3, 8), (2, 4, 2, 5, 128),
              (1, 3, 3, 17, 8), (1, 4, 1, 64, 128), (2, 2, 2, 129, 2), (1, 8, 2, 40, 16)]


def pin_bwd_library(bref, shapes=LIB_SHAPES):
    for t, (B, Hq, Hkv, N, D) in enumerate(shapes):
        q, k = rnd(400 + t, (B, Hq, N, D)), rnd(500 + t, (B, Hkv, N, D))
        v, do = rnd(600 + t, (B, Hkv, N, D)), rnd(700 + t, (B, Hq, N, D))
        for causal in (False, True):
            got = bref(q, k, v, do, causal, SCALE)
            exp = torch_grads_f64(q, k, v, do, causal, SCALE)
            for name, a, e in zip(("dQ", "dK", "dV"), got, exp):
                close(a, e, tol=1e-11, what=f"torch autograd {name} {B,Hq,Hkv,N,D} c={causal}")


# --------------------------------------------------------------- hand-derived
def pin_bwd_hand_example(bref):
    """Scalar head (D = 1), keys k = (0, 1), values v = (1, 3), scale 1, two query
    rows with q = 1 and dO = 1.  With p = (1, e)/(1 + e):
    dO_i/ds_i1 = -dO_i/ds_i0 = p0 p1 (v1 - v0) = 2e/(1+e)^2 =: c, so per row
    dQ = k1 c = c, dK = (-c, c) * q, dV = p.  Non-causal: dK, dV sum both rows.
    Causal: row 0 sees only key 0 (p = 1, every dS = 0), row 1 as above."""
    q = bf(np.ones((1, 1, 2, 1)))
    k = bf(np.array([0.0, 1.0]).reshape(1, 1, 2, 1))
    v = bf(np.array([1.0, 3.0]).reshape(1, 1, 2, 1))
    do = bf(np.ones((1, 1, 2, 1)))
    e = math.e
    c = 2 * e / (1 + e) ** 2
    p = np.array([1.0, e]) / (1 + e)
    dq, dk, dv = bref(q, k, v, do, False, 1.0)
    close(dq.ravel(), [c, c], what="hand dQ")
    close(dk.ravel(), [-2 * c, 2 * c], what="hand dK")
    close(dv.ravel(), 2 * p, what="hand dV")
    dq, dk, dv = bref(q, k, v, do, True, 1.0)
    close(dq.ravel(), [0.0, c], what="hand causal dQ")
    close(dk.ravel(), [-c, c], what="hand causal dK")
    close(dv.ravel(), [1.0 + p[0], p[1]], what="hand causal dV")


# ---------------------------------------------------------------- closed forms
def pin_bwd_uniform(bref):
    """Q = 0: every allowed weight is 1/n_i.  Then dK = 0, dV_j = sum over rows i
    that see j of dO_i / n_i, and dQ_i = (scale/n_i) sum_j (dO_i.V_j - mean) K_j
    (mean over J_i of dO_i.V_j)."""
    B, Hq, Hkv, N, D = 1, 4, 2, 19, 8
    k, v, do = rnd(11, (B, Hkv, N, D)), rnd(12, (B, Hkv, N, D)), rnd(13, (B, Hq, N, D))
    q = np.zeros((B, Hq, N, D), np.uint16)
    kf, vf, dof = bits_to64(k), bits_to64(v), bits_to64(do)
    g = Hq // Hkv
    for causal in (False, True):
        dq, dk, dv = bref(q, k, v, do, causal, SCALE)
        assert np.all(dk == 0.0), "Q = 0 must give dK = 0"
        edq = np.zeros_like(dq)
        edv = np.zeros_like(dv)
        for b in range(B):
            for h in range(Hq):
                kv = h // g
                for i in range(N):
                    n = i + 1 if causal else N
                    dp = vf[b, kv, :n] @ dof[b, h, i]
                    edq[b, h, i] = SCALE / n * ((dp - dp.mean()) @ kf[b, kv, :n])
                    edv[b, kv, :n] += dof[b, h, i] / n
        close(dq, edq, what=f"uniform dQ causal={causal}")
        close(dv, edv, what=f"uniform dV causal={causal}")


# ------------------------------------------------------------------ invariants
def pin_bwd_sums(bref):
    """Each row of dS sums to zero, so sum_j dK_j = 0; each row of P sums to one,
    so sum_j dV_j = sum of dO over the group's rows; L depends on Q and K only
    through Q K^T, so <Q, dQ> = <K, dK>; and <V, dV> = <dO, O> with O from the
    forward oracle."""
    for (B, Hq, Hkv, N, D) in ((2, 4, 2, 33, 16), (1, 3, 1, 50, 64)):
        q, k = rnd(21, (B, Hq, N, D)), rnd(22, (B, Hkv, N, D))
        v, do = rnd(23, (B, Hkv, N, D)), rnd(24, (B, Hq, N, D))
        g = Hq // Hkv
        for causal in (False, True):
            dq, dk, dv = bref(q, k, v, do, causal, SCALE)
            o, _ = _fwd(q, k, v, causal, SCALE)
            dof = bits_to64(do)
            scale_k = np.abs(dk).sum(axis=2).max()
            close(dk.sum(axis=2) / scale_k, np.zeros((B, Hkv, D)), tol=1e-13,
                  what="sum_j dK_j = 0")
            close(dv.sum(axis=2), dof.reshape(B, Hkv, g, N, D).sum(axis=(2, 3)),
                  what="sum_j dV_j = sum dO")
            close(np.sum(bits_to64(q) * dq), np.sum(bits_to64(k) * dk), what="<Q,dQ> = <K,dK>")
            close(np.sum(bits_to64(v) * dv), np.sum(dof * o), what="<V,dV> = <dO,O>")


def pin_bwd_key_shift(bref):
    """Adding one vector u to every key shifts each row's scores by a constant:
    P, and so every gradient, is unchanged (the dK shift term is scale * u *
    sum_j dS_ij = 0)."""
    B, H, N, D = 1, 2, 23, 32
    g = np.random.default_rng(9)
    q = bf(g.integers(-16, 17, (B, H, N, D)) / 8.0)
    k = bf(g.integers(-16, 17, (B, H, N, D)) / 8.0)
    u = g.integers(-16, 17, (D,)) / 8.0
    k2 = bf(bits_to64(k) + u)
    v, do = rnd(31, (B, H, N, D)), rnd(32, (B, H, N, D))
    for causal in (False, True):
        a = bref(q, k, v, do, causal, SCALE)
        b = bref(q, k2, v, do, causal, SCALE)
        for name, x, y in zip(("dQ", "dK", "dV"), a, b):
            close(y, x, tol=1e-11, what=f"key shift {name} causal={causal}")


def pin_bwd_gqa(bref):
    """GQA == MHA with K/V repeated per group: dQ identical, and dK, dV of a shared
    head equal the sum over its group of the repeated heads' gradients."""
    for (Hq, Hkv) in ((8, 2), (6, 1)):
        B, N, D = 2, 17, 16
        q, k = rnd(41, (B, Hq, N, D)), rnd(42, (B, Hkv, N, D))
        v, do = rnd(43, (B, Hkv, N, D)), rnd(44, (B, Hq, N, D))
        g = Hq // Hkv
        for causal in (False, True):
            dq1, dk1, dv1 = bref(q, k, v, do, causal, SCALE)
            dq2, dk2, dv2 = bref(q, np.repeat(k, g, axis=1), np.repeat(v, g, axis=1), do,
                                 causal, SCALE)
            assert np.array_equal(dq1, dq2), f"GQA {Hq}/{Hkv} dQ != MHA dQ"
            close(dk1, dk2.reshape(B, Hkv, g, N, D).sum(axis=2), what="GQA dK = group sum")
            close(dv1, dv2.reshape(B, Hkv, g, N, D).sum(axis=2), what="GQA dV = group sum")


def pin_bwd_causal_structure(bref):
    """Causal: row 0 has one key (P = 1, dS = 0) so dQ_0 = 0 exactly; dQ of rows
    <= i ignores K, V rows > i; dK_j, dV_j ignore Q, dO rows < j (only rows >= j
    see key j); the last key's dV is P_{N-1,N-1} dO_{N-1}."""
    B, H, N, D = 1, 2, 26, 16
    q, k, v, do = (rnd(51 + t, (B, H, N, D)) for t in range(4))
    dq, dk, dv = bref(q, k, v, do, True, SCALE)
    assert np.all(dq[:, :, 0] == 0.0), "causal dQ of row 0 must be 0"
    i = 9
    k2, v2 = k.copy(), v.copy()
    k2[:, :, i + 1:] = rnd(55, k2[:, :, i + 1:].shape, 3.0)
    v2[:, :, i + 1:] = rnd(56, v2[:, :, i + 1:].shape)
    dq2, _, _ = bref(q, k2, v2, do, True, SCALE)
    assert np.array_equal(dq[:, :, :i + 1], dq2[:, :, :i + 1]), "future keys changed past dQ"
    q3, do3 = q.copy(), do.copy()
    q3[:, :, :i] = rnd(57, q3[:, :, :i].shape, 3.0)
    do3[:, :, :i] = rnd(58, do3[:, :, :i].shape)
    _, dk3, dv3 = bref(q3, k, v, do3, True, SCALE)
    assert np.array_equal(dk[:, :, i:], dk3[:, :, i:]) and \
        np.array_equal(dv[:, :, i:], dv3[:, :, i:]), "earlier rows changed a later key's grads"
    assert not np.array_equal(dk[:, :, :i], dk3[:, :, :i]), "rows before i ignored"
    _, lse = _fwd(q, k, v, True, SCALE)
    s = SCALE * np.sum(bits_to64(q)[:, :, -1] * bits_to64(k)[:, :, -1], axis=-1)
    plast = np.exp(s - lse[:, :, -1])
    close(dv[:, :, -1], plast[..., None] * bits_to64(do)[:, :, -1], what="last key dV")


def pin_bwd_rows_subset(bref):
    """The dQ-rows mode returns exactly those rows of the full dQ."""
    B, Hq, Hkv, N, D = 2, 4, 2, 21, 16
    q, k = rnd(61, (B, Hq, N, D)), rnd(62, (B, Hkv, N, D))
    v, do = rnd(63, (B, Hkv, N, D)), rnd(64, (B, Hq, N, D))
    rows = np.array([0, 5, 20, 21, 100, B * Hq * N - 1, 7], np.int64)
    for causal in (False, True):
        dq, _, _ = bref(q, k, v, do, causal, SCALE)
        dqs = bref(q, k, v, do, causal, SCALE, rows=rows)
        assert np.array_equal(dqs, dq.reshape(-1, D)[rows]), "dQ row subset"


def pin_bwd_keys_subset(bref):
    """The key-subset mode returns exactly those key rows of the full dK, dV (and
    of their error-scale sums)."""
    B, Hq, Hkv, N, D = 2, 6, 3, 19, 16
    q, k = rnd(65, (B, Hq, N, D)), rnd(66, (B, Hkv, N, D))
    v, do = rnd(67, (B, Hkv, N, D)), rnd(68, (B, Hq, N, D))
    # the second list holds only late keys of each panel it touches, so the
    # causal key mode skips the rows before them
    key_lists = (np.array([0, 18, 19, 40, B * Hkv * N - 1, 3], np.int64),
                 np.array([17, 18, 15, 19 + 12, 2 * 19 + 16, 5 * 19 + 18], np.int64))
    for causal in (False, True):
        _, dk, dv, _, mk, mv = bref(q, k, v, do, causal, SCALE, mags=True)
        for keys in key_lists:
            dks, dvs, mks, mvs = bref(q, k, v, do, causal, SCALE, keys=keys, mags=True)
            for full, sub in ((dk, dks), (dv, dvs), (mk, mks), (mv, mvs)):
                assert np.array_equal(sub, full.reshape(-1, D)[keys]), "key subset"


def pin_bwd_error_scales(bref):
    """The error-scale sums bound each gradient (triangle inequality), and equal
    it where every term is non-negative: mag_dV = dV when dO >= 0."""
    B, Hq, Hkv, N, D = 1, 4, 2, 30, 16
    q, k = rnd(71, (B, Hq, N, D)), rnd(72, (B, Hkv, N, D))
    v = rnd(73, (B, Hkv, N, D))
    do = rnd(74, (B, Hq, N, D))
    for causal in (False, True):
        dq, dk, dv, mq, mk, mv = bref(q, k, v, do, causal, SCALE, mags=True)
        for name, g, m in (("dQ", dq, mq), ("dK", dk, mk), ("dV", dv, mv)):
            assert np.all(m >= np.abs(g) * (1 - 1e-12)), f"{name} error scale below |grad|"
        dq2, mq2 = bref(q, k, v, do, causal, SCALE, rows=np.arange(B * Hq * N), mags=True)
        assert np.array_equal(mq2, mq.reshape(-1, D)), "dQ error scale in rows mode"
        dop = bf(np.abs(bits_to64(do)))
        _, _, dvp, _, _, mvp = bref(q, k, v, dop, causal, SCALE, mags=True)
        close(mvp, dvp, tol=1e-14, what="mag_dV = dV for dO >= 0")


ALL_PINS = [pin_bwd_finite_difference, pin_bwd_library, pin_bwd_hand_example,
            pin_bwd_uniform, pin_bwd_sums, pin_bwd_key_shift, pin_bwd_gqa,
            pin_bwd_causal_structure, pin_bwd_rows_subset, pin_bwd_keys_subset,
            pin_bwd_error_scales]
