"""Checks that pin the fp64 oracle to facts other than itself.

Each ``pin_*`` takes ``ref(q, k, v, causal, scale, rows=None) -> (o, lse)``
(bf16 bit arrays in, float64 out) and raises AssertionError when the result
contradicts a closed form, an invariant, a library routine or a value printed
on the pages.  They are used on the real oracle (test_oracle_pins.py) and on
copies of it with planted mistakes (test_oracle_mutations.py), where at least
one pin must fail for every planted mistake.

The definition being pinned: page "GPU注意力算子性能优化" (QiMeng-Attention),
section 1 (softmax(Q K^T / sqrt(d_k)) V); page "AVO算法优化Transformer注意力机制
性能解析", section 3.1 (max-subtracted softmax, scale folded into the scores);
the QiMeng page, section 3.2 (K/V shared by a group of query heads).
"""
from __future__ import annotations

import math

import numpy as np
import scipy.special
import torch

from synth import bf16_bits_to_f32, f32_to_bf16_bits, normal_bf16

TIGHT = 1e-12


def bf(x) -> np.ndarray:
    """float array -> bf16 bits; asserts the values are exactly representable."""
    x = np.asarray(x, dtype=np.float64)
    bits = f32_to_bf16_bits(x.astype(np.float32))
    assert np.array_equal(bits_to64(bits), x), "fixture value not exact in bf16"
    return bits


def bits_to64(b) -> np.ndarray:
    return bf16_bits_to_f32(b).astype(np.float64)


def rnd(seed, shape, mult=1.0):
    return normal_bf16(seed, shape, mult)


def close(a, b, tol=TIGHT, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite result"
    err = np.max(np.abs(a - b) / (1.0 + np.abs(b))) if a.size else 0.0
    assert err <= tol, f"{what}: max rel err {err:.3e} > {tol:.1e}"


SCALE = float(np.float32(1.0 / math.sqrt(128.0)))


# ---------------------------------------------------------------- closed forms
def pin_identical_keys(ref):
    """All keys equal -> every allowed score equal -> O_i = mean of V over J_i,
    LSE_i = s_i + ln|J_i|."""
    B, H, N, D = 1, 2, 37, 16
    q = rnd(11, (B, H, N, D))
    k1 = rnd(12, (B, H, 1, D))
    k = np.repeat(k1, N, axis=2)
    v = rnd(13, (B, H, N, D))
    qf, kf, vf = bits_to64(q), bits_to64(k), bits_to64(v)
    s = SCALE * np.einsum("bhid,bhd->bhi", qf, kf[:, :, 0, :])
    for causal in (False, True):
        o, lse = ref(q, k, v, causal, SCALE)
        if causal:
            cnt = np.arange(1, N + 1, dtype=np.float64)
            mean = np.cumsum(vf, axis=2) / cnt[None, None, :, None]
        else:
            cnt = np.full(N, float(N))
            mean = np.broadcast_to(vf.mean(axis=2, keepdims=True), vf.shape)
        close(o, mean, what=f"identical keys O causal={causal}")
        close(lse, s + np.log(cnt)[None, None, :], what=f"identical keys LSE causal={causal}")


def pin_dominant_score(ref):
    """One key whose score beats every other by > 80 nats selects its V row."""
    B, H, N, D = 1, 1, 50, 8
    jstar = 23
    q = np.zeros((B, H, N, D)); q[..., 0] = 16.0
    k = np.zeros((B, H, N, D))
    k[..., 0] = bits_to64(rnd(21, (B, H, N))) * 0.125
    k[..., 1:] = bits_to64(rnd(22, (B, H, N, D - 1)))
    k[0, 0, jstar, 0] = 64.0
    kb = f32_to_bf16_bits(k.astype(np.float32))
    qb = bf(q)
    v = rnd(23, (B, H, N, D))
    vf = bits_to64(v)
    kf = bits_to64(kb)
    sstar = SCALE * 16.0 * 64.0
    o, lse = ref(qb, kb, v, False, SCALE)
    close(o, np.broadcast_to(vf[:, :, jstar:jstar + 1, :], o.shape), tol=1e-15,
          what="dominant score O")
    rest = SCALE * 16.0 * kf[0, 0, :, 0]
    exact_lse = sstar + np.log(np.sum(np.exp(rest - sstar)))
    close(lse[0, 0], np.full(N, exact_lse), what="dominant score LSE")
    # causal: rows before j* cannot see j*; rows from j* on select it
    oc, lsec = ref(qb, kb, v, True, SCALE)
    close(oc[0, 0, jstar:], np.broadcast_to(vf[0, 0, jstar], (N - jstar, D)), tol=1e-15,
          what="causal dominant O")
    assert np.all(np.abs(oc[0, 0, :jstar] - vf[0, 0, jstar]).max(axis=-1) > 1e-3), \
        "causal: a row before the dominant key selected it"
    assert np.all(lsec[0, 0, :jstar] < sstar - 50), "causal: early rows saw a future key"


def pin_causal_row0(ref):
    """Causal row 0 sees only key 0: O[0] = V[0] exactly, LSE[0] = scale * q0.k0."""
    B, H, N, D = 2, 3, 19, 32
    q, k, v = rnd(31, (B, H, N, D)), rnd(32, (B, H, N, D)), rnd(33, (B, H, N, D))
    o, lse = ref(q, k, v, True, SCALE)
    assert np.array_equal(o[:, :, 0, :], bits_to64(v)[:, :, 0, :]), "causal row 0 != V[0]"
    s00 = SCALE * np.sum(bits_to64(q)[:, :, 0, :] * bits_to64(k)[:, :, 0, :], axis=-1)
    close(lse[:, :, 0], s00, what="causal row 0 LSE")


def pin_probabilities(ref):
    """With one-hot V rows (V_j = e_j, D >= N) the output row is the probability
    row itself: non-negative, sums to 1, and equals scipy's softmax of the
    scaled score row (a library routine on library-computed scores)."""
    B, H, N, D = 1, 2, 24, 32
    q, k = rnd(41, (B, H, N, D)), rnd(42, (B, H, N, D))
    v = np.zeros((B, H, N, D)); v[:, :, np.arange(N), np.arange(N)] = 1.0
    vb = bf(v)
    sc = SCALE * np.matmul(bits_to64(q), np.swapaxes(bits_to64(k), -1, -2))
    for causal in (False, True):
        o, _ = ref(q, k, vb, causal, SCALE)
        p = o[..., :N]
        assert np.all(o[..., N:] == 0.0), "mass outside the key range"
        assert np.all(p >= 0.0), "negative probability"
        close(p.sum(axis=-1), np.ones((B, H, N)), what="rows sum to 1")
        s = sc.copy()
        if causal:
            s[..., np.triu_indices(N, 1)[0], np.triu_indices(N, 1)[1]] = -np.inf
        close(p, scipy.special.softmax(s, axis=-1), what=f"probabilities causal={causal}")


def pin_constant_v(ref):
    """V = c everywhere -> O = c (normalisation)."""
    B, H, N, D = 1, 2, 33, 16
    q, k = rnd(51, (B, H, N, D), 3.0), rnd(52, (B, H, N, D), 3.0)
    v = bf(np.full((B, H, N, D), -2.75))
    for causal in (False, True):
        o, _ = ref(q, k, v, causal, SCALE)
        close(o, np.full(o.shape, -2.75), what="constant V")


def pin_uniform(ref):
    """Q = 0, or scale = 0 -> uniform weights: O = mean V over J_i, LSE = ln|J_i|."""
    B, H, N, D = 1, 2, 29, 8
    q, k, v = rnd(61, (B, H, N, D)), rnd(62, (B, H, N, D)), rnd(63, (B, H, N, D))
    vf = bits_to64(v)
    zero_q = np.zeros_like(q)
    for causal in (False, True):
        cnt = np.arange(1, N + 1, dtype=np.float64) if causal else np.full(N, float(N))
        mean = (np.cumsum(vf, axis=2) / cnt[None, None, :, None]) if causal else \
            np.broadcast_to(vf.mean(axis=2, keepdims=True), vf.shape)
        for qq, sc in ((zero_q, SCALE), (q, 0.0)):
            o, lse = ref(qq, k, v, causal, sc)
            close(o, mean, what="uniform O")
            close(lse, np.broadcast_to(np.log(cnt), lse.shape), what="uniform LSE")


def pin_single_key(ref):
    """N = 1: O = V[0], LSE = the one score."""
    q, k, v = rnd(71, (2, 4, 1, 128)), rnd(72, (2, 2, 1, 128)), rnd(73, (2, 2, 1, 128))
    for causal in (False, True):
        o, lse = ref(q, k, v, causal, SCALE)
        kv_of_h = np.arange(4) // 2
        assert np.array_equal(o, bits_to64(v)[:, kv_of_h]), "N=1 O != V"
        s = SCALE * np.sum(bits_to64(q) * bits_to64(k)[:, kv_of_h], axis=-1)
        close(lse, s, what="N=1 LSE")


def pin_hand_example(ref):
    """Hand-derived two-key case: q = [1], keys 0 and 1, values 1 and 3, scale 1:
    p = (1, e)/(1 + e), O = (1 + 3e)/(1 + e), LSE = ln(1 + e)."""
    q = bf(np.ones((1, 1, 2, 1)))
    k = bf(np.array([0.0, 1.0]).reshape(1, 1, 2, 1))
    v = bf(np.array([1.0, 3.0]).reshape(1, 1, 2, 1))
    o, lse = ref(q, k, v, False, 1.0)
    e = math.e
    close(o[0, 0, :, 0], [(1 + 3 * e) / (1 + e)] * 2, what="hand example O")
    close(lse[0, 0], [math.log1p(e)] * 2, what="hand example LSE")
    oc, lsec = ref(q, k, v, True, 1.0)
    close(oc[0, 0, :, 0], [1.0, (1 + 3 * e) / (1 + e)], what="hand example causal O")
    close(lsec[0, 0], [0.0, math.log1p(e)], what="hand example causal LSE")


# ------------------------------------------------------------- library routine
def torch_sdpa_f64(q, k, v, causal, scale):
    """torch's CPU scaled_dot_product_attention in float64, K/V heads repeated per group."""
    g = q.shape[1] // k.shape[1]
    qt = torch.from_numpy(bits_to64(q))
    kt = torch.from_numpy(bits_to64(k)).repeat_interleave(g, dim=1)
    vt = torch.from_numpy(bits_to64(v)).repeat_interleave(g, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=bool(causal),
                                                         scale=float(scale))
    s = float(scale) * np.matmul(qt.numpy(), np.swapaxes(kt.numpy(), -1, -2))
    if causal:
        n = s.shape[-1]
        s[..., np.triu_indices(n, 1)[0], np.triu_indices(n, 1)[1]] = -np.inf
    return o.numpy(), scipy.special.logsumexp(s, axis=-1)


LIB_SHAPES = [(1, 1, 1, 1, 1), (1, 1, 1, 2, 2), (1, 2, 1, 3, 8), (2, 4, 2, 5, 128),
              (1, 3, 3, 17, 8), (1, 4, 1, 64, 128), (2, 2, 2, 129, 2), (1, 8, 2, 100, 128)]


def pin_library(ref, shapes=LIB_SHAPES):
    """Whole formula vs torch's fp64 CPU SDPA and scipy's logsumexp."""
    for t, (B, Hq, Hkv, N, D) in enumerate(shapes):
        q = rnd(100 + t, (B, Hq, N, D))
        k = rnd(200 + t, (B, Hkv, N, D))
        v = rnd(300 + t, (B, Hkv, N, D))
        for causal in (False, True):
            o, lse = ref(q, k, v, causal, SCALE)
            eo, else_ = torch_sdpa_f64(q, k, v, causal, SCALE)
            close(o, eo, tol=1e-12, what=f"torch sdpa {B,Hq,Hkv,N,D} causal={causal}")
            close(lse, else_, tol=1e-12, what=f"logsumexp {B,Hq,Hkv,N,D} causal={causal}")


# ------------------------------------------------------------------ invariants
def pin_gqa_equals_repeated_mha(ref):
    """GQA/MQA == MHA with each K/V head repeated for its group (bitwise)."""
    for (Hq, Hkv) in ((8, 2), (6, 1), (4, 4)):
        B, N, D = 2, 21, 16
        q, k, v = rnd(81, (B, Hq, N, D)), rnd(82, (B, Hkv, N, D)), rnd(83, (B, Hkv, N, D))
        g = Hq // Hkv
        kr, vr = np.repeat(k, g, axis=1), np.repeat(v, g, axis=1)
        for causal in (False, True):
            o1, l1 = ref(q, k, v, causal, SCALE)
            o2, l2 = ref(q, kr, vr, causal, SCALE)
            assert np.array_equal(o1, o2) and np.array_equal(l1, l2), f"GQA {Hq}/{Hkv} != MHA"


def pin_key_shift(ref):
    """Adding one vector u to every key leaves O unchanged and adds scale*q.u to
    LSE (the softmax is shift invariant).  Values are multiples of 1/8 so K + u
    is exact in bf16.  The second case shifts every score by ~1.5e3 nats, which
    overflows exp() unless the row max is subtracted first."""
    B, H, N, D = 1, 2, 31, 64
    g = np.random.default_rng(5)
    k = bf(g.integers(-16, 17, (B, H, N, D)) / 8.0)
    v = rnd(91, (B, H, N, D))
    cases = (
        (bf(g.integers(-16, 17, (B, H, N, D)) / 8.0), g.integers(-16, 17, (D,)) / 8.0),
        (bf(g.integers(1, 17, (B, H, N, D)) * 4.0), np.full(D, 8.0)),
    )
    for q, u in cases:
        k2 = bf(bits_to64(k) + u)
        shift = SCALE * np.einsum("bhid,d->bhi", bits_to64(q), u)
        for causal in (False, True):
            o1, l1 = ref(q, k, v, causal, SCALE)
            o2, l2 = ref(q, k2, v, causal, SCALE)
            close(o2, o1, tol=1e-11, what=f"shift O max|shift|={np.abs(shift).max():.0f}")
            close(l2, l1 + shift, tol=1e-11, what="shift LSE")


def pin_key_permutation(ref):
    """Non-causal: permuting (K_j, V_j) pairs jointly leaves O and LSE unchanged."""
    B, H, N, D = 1, 2, 40, 16
    q, k, v = rnd(101, (B, H, N, D)), rnd(102, (B, H, N, D)), rnd(103, (B, H, N, D))
    perm = np.random.default_rng(3).permutation(N)
    o1, l1 = ref(q, k, v, False, SCALE)
    o2, l2 = ref(q, k[:, :, perm], v[:, :, perm], False, SCALE)
    close(o2, o1, what="permutation O")
    close(l2, l1, what="permutation LSE")


def pin_causal_future(ref):
    """Causal: changing keys/values after row i leaves rows 0..i unchanged (bitwise)."""
    B, H, N, D = 1, 2, 30, 16
    q, k, v = rnd(111, (B, H, N, D)), rnd(112, (B, H, N, D)), rnd(113, (B, H, N, D))
    i = 12
    k2, v2 = k.copy(), v.copy()
    k2[:, :, i + 1:] = rnd(114, k2[:, :, i + 1:].shape, 4.0)
    v2[:, :, i + 1:] = rnd(115, v2[:, :, i + 1:].shape)
    o1, l1 = ref(q, k, v, True, SCALE)
    o2, l2 = ref(q, k2, v2, True, SCALE)
    assert np.array_equal(o1[:, :, :i + 1], o2[:, :, :i + 1]), "future keys changed the past"
    assert np.array_equal(l1[:, :, :i + 1], l2[:, :, :i + 1]), "future keys changed past LSE"
    assert not np.array_equal(o1[:, :, i + 1:], o2[:, :, i + 1:]), "later rows ignored their keys"


def pin_causal_prefix(ref):
    """Causal rows 0..M-1 of N tokens == causal attention on the first M tokens."""
    B, H, N, D, M = 1, 2, 45, 16, 17
    q, k, v = rnd(121, (B, H, N, D)), rnd(122, (B, H, N, D)), rnd(123, (B, H, N, D))
    o1, l1 = ref(q, k, v, True, SCALE)
    o2, l2 = ref(q[:, :, :M], k[:, :, :M], v[:, :, :M], True, SCALE)
    assert np.array_equal(o1[:, :, :M], o2) and np.array_equal(l1[:, :, :M], l2), "prefix"


def pin_row_subset(ref):
    """Asking for a subset of rows returns exactly those rows of the full result."""
    B, Hq, Hkv, N, D = 2, 4, 2, 23, 32
    q, k, v = rnd(131, (B, Hq, N, D)), rnd(132, (B, Hkv, N, D)), rnd(133, (B, Hkv, N, D))
    rows = np.array([0, 5, 22, 23, 99, B * Hq * N - 1, 7], dtype=np.int64)
    for causal in (False, True):
        o, l = ref(q, k, v, causal, SCALE)
        os_, ls = ref(q, k, v, causal, SCALE, rows=rows)
        assert np.array_equal(os_, o.reshape(-1, D)[rows]) and \
            np.array_equal(ls, l.reshape(-1)[rows]), "row subset"


# ---------------------------------------------------------------- non-finite inputs
NAN_BITS, PINF_BITS, NINF_BITS = 0x7FC0, 0x7F80, 0xFF80


def pin_nonfinite(ref):
    """Non-finite inputs follow the formula in IEEE arithmetic (limits that hold
    for any correct evaluation of it):
      * NaN in q_i -> row i all NaN (O and LSE), every other row unchanged;
      * NaN or +inf in V_j[d] -> O_i[d] NaN or +inf exactly for the rows that see
        key j (each has weight > 0), every other element unchanged; +inf at
        key j1 and -inf at key j2 > j1 of one column -> causal rows in
        [j1, j2) +inf, rows from j2 on NaN;
      * a -inf score of key j (q_i . k_j = -inf) gives it weight 0: row i equals
        attention over the keys without j;
      * a row whose scores are all -inf is NaN (max -inf, exp(-inf + inf) NaN);
        a +inf score makes its row NaN (exp(inf - inf))."""
    B, H, N, D = 1, 2, 24, 16
    q, k, v = rnd(141, (B, H, N, D)), rnd(142, (B, H, N, D)), rnd(143, (B, H, N, D))
    for causal in (False, True):
        o0, l0 = ref(q, k, v, causal, SCALE)
        sees = (np.arange(N)[:, None] >= np.arange(N)[None, :]) if causal else np.ones((N, N), bool)
        # NaN in q
        q1 = q.copy()
        q1[0, 1, 9, 3] = NAN_BITS
        o1, l1 = ref(q1, k, v, causal, SCALE)
        assert np.all(np.isnan(o1[0, 1, 9])) and np.isnan(l1[0, 1, 9]), "NaN query row"
        keep = np.ones((B, H, N), bool)
        keep[0, 1, 9] = False
        assert np.array_equal(o1[keep], o0[keep]) and np.array_equal(l1[keep], l0[keep]), "NaN row spread"
        # NaN / inf in V
        for bits, test in ((NAN_BITS, np.isnan), (PINF_BITS, np.isposinf)):
            v2 = v.copy()
            v2[0, 0, 13, 5] = bits
            o2, l2 = ref(q, k, v2, causal, SCALE)
            hit = np.zeros((B, H, N, D), bool)
            hit[0, 0, sees[:, 13], 5] = True
            assert np.all(test(o2[hit])), "non-finite V must reach every row that sees its key"
            assert np.array_equal(o2[~hit], o0[~hit]) and np.array_equal(l2, l0), "non-finite V spread"
        # +inf then -inf in one column
        v3 = v.copy()
        v3[0, 1, 4, 7] = PINF_BITS
        v3[0, 1, 15, 7] = NINF_BITS
        o3, _ = ref(q, k, v3, causal, SCALE)
        col = o3[0, 1, :, 7]
        if causal:
            assert np.all(np.isfinite(col[:4])) and np.all(np.isposinf(col[4:15])) and np.all(np.isnan(col[15:]))
        else:
            assert np.all(np.isnan(col)), "+inf and -inf of one column give NaN"
    # a -inf score drops its key: key j holds -inf in a dimension where row i's
    # query is +1, so s_ij = -inf; row i then equals torch's fp64 SDPA and
    # scipy's logsumexp over the other keys
    q4, k4 = q.copy(), k.copy()
    j, i = 6, 20
    q4[0, 0, i, 2] = bf([1.0])[0]
    k4[0, 0, j, 2] = NINF_BITS
    o4, l4 = ref(q4, k4, v, False, SCALE)
    others = [x for x in range(N) if x != j]
    qi = torch.from_numpy(bits_to64(q4[0, 0, i:i + 1]))
    ko = torch.from_numpy(bits_to64(k4[0, 0, others]))
    vo = torch.from_numpy(bits_to64(v[0, 0, others]))
    eo = torch.nn.functional.scaled_dot_product_attention(qi, ko, vo, scale=SCALE)
    el = scipy.special.logsumexp(SCALE * (qi.numpy() @ ko.numpy().T), axis=-1)
    close(o4[0, 0, i], eo.numpy()[0], tol=1e-12, what="-inf score drops its key")
    close(l4[0, 0, i], el[0], tol=1e-12, what="-inf score drops its key (LSE)")
    # the dropped key still takes part in the sum: 0 * NaN is NaN
    v4 = v.copy()
    v4[0, 0, j, 1] = NAN_BITS
    o4n, _ = ref(q4, k4, v4, False, SCALE)
    assert np.isnan(o4n[0, 0, i, 1]), "a zero weight times NaN is NaN"
    assert np.array_equal(np.delete(o4n[0, 0, i], 1), np.delete(o4[0, 0, i], 1)), "zero-weight NaN spread"
    # all -inf row, and a +inf score
    q6, k6 = q.copy(), k.copy()
    k6[0, 0, :, 11] = bf([-1.0])[0]
    q6[0, 0, 3, 11] = PINF_BITS       # every score of row 3 is -inf
    k6[0, 1, 8, 0] = PINF_BITS
    q6[0, 1, 17, 0] = bf([1.0])[0]    # score of key 8 for row 17 is +inf
    for causal in (False, True):
        o6, l6 = ref(q6, k6, v, causal, SCALE)
        assert np.all(np.isnan(o6[0, 0, 3])) and np.isnan(l6[0, 0, 3]), "all -inf row must be NaN"
        assert np.all(np.isnan(o6[0, 1, 17])) and np.isnan(l6[0, 1, 17]), "+inf score row must be NaN"
        assert np.all(np.isfinite(o6[0, 0, :3])), "other rows of the all -inf head stay finite"


ALL_PINS = [pin_identical_keys, pin_dominant_score, pin_causal_row0, pin_probabilities,
            pin_constant_v, pin_uniform, pin_single_key, pin_hand_example, pin_library,
            pin_gqa_equals_repeated_mha, pin_key_shift, pin_key_permutation,
            pin_causal_future, pin_causal_prefix, pin_row_subset, pin_nonfinite]
