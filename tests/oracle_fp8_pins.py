"""Checks that pin the fp64 FP8 (e4m3) oracle to facts other than itself.

Each ``pin_*`` takes ``(fref, dec)``: ``fref(q8, k8, v8, dq, dk, dv, causal, scale,
rows=None, mags=None)`` is the oracle forward on e4m3 codes with per-tensor
descales (see ``oracle.attn_fp8_ref``) and ``dec(codes)`` its code-to-value rule.
A pin raises AssertionError when a result contradicts the OCP e4m3 format (as
torch's ``float8_e4m3fn`` implements it and as the format's definition fixes
single values), the separately pinned bf16-input forward oracle, torch's fp64
SDPA on the decoded tensors, or a closed form.  They run on the real oracle
(test_oracle_fp8_pins.py) and on copies with planted mistakes
(test_oracle_fp8_mutations.py).

What is pinned: the forward's definition (page "GPU注意力算子性能优化"
(QiMeng-Attention), section 1) evaluated on the tensors that FP8 codes and
per-tensor scales stand for (FP8 matrix products with fp32 softmax and
accumulation: page "注意力机制的本质与计算挑战", section 3; the QiMeng page,
section 3.1.1), and the error-scale sum the GPU parity tolerance is built from.
"""
from __future__ import annotations

import math

import numpy as np
import scipy.special
import torch

import oracle
from synth import f32_to_bf16_bits, normal_e4m3
from tests.oracle_pins import SCALE, close


def torch_decode(codes) -> np.ndarray:
    """e4m3 codes -> float64 through torch's float8_e4m3fn dtype."""
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def _codes(seed, shape, descale=2.0 ** -5):
    return normal_e4m3(seed, shape, descale)


# ---------------------------------------------------------------- the format
def pin_decode_matches_torch(fref, dec):
    """All 256 codes decode as torch's float8_e4m3fn does (NaN where it is NaN,
    signed zeros included)."""
    c = np.arange(256, dtype=np.uint8)
    a, b = dec(c), torch_decode(c)
    assert np.array_equal(np.isnan(a), np.isnan(b)), "NaN codes differ from float8_e4m3fn"
    ok = ~np.isnan(b)
    assert np.array_equal(a[ok], b[ok]), "decoded values differ from float8_e4m3fn"
    assert np.array_equal(np.signbit(a[ok]), np.signbit(b[ok])), "signs differ"


def pin_decode_format_values(fref, dec):
    """Values the e4m3 definition fixes: 1.0 = 0x38, largest finite 448 = 0x7E,
    smallest normal 2^-6 = 0x08, smallest subnormal 2^-9 = 0x01, largest
    subnormal 7 * 2^-9 = 0x07, NaN only at 0x7F / 0xFF, sign bit 0x80, and the
    positive codes 0x00..0x7E strictly increasing."""
    want = {0x38: 1.0, 0x7E: 448.0, 0x08: 2.0 ** -6, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9,
            0x40: 2.0, 0x3C: 1.5, 0xB8: -1.0, 0xFE: -448.0, 0x00: 0.0}
    got = dec(np.array(list(want), dtype=np.uint8))
    assert np.array_equal(got, np.array(list(want.values()))), f"format values: {got}"
    v = dec(np.arange(256, dtype=np.uint8))
    nan = np.flatnonzero(np.isnan(v))
    assert list(nan) == [0x7F, 0xFF], f"NaN codes {nan}"
    assert np.all(np.diff(v[:127]) > 0), "positive codes not increasing"
    assert np.array_equal(v[128:255], -v[:127]), "negative codes not mirrored"


# ---------------------------------------------------------------- the forward
def pin_equals_bf16_oracle(fref, dec):
    """With power-of-two descales every decoded value is exact in bf16, so the
    result equals the (separately pinned) bf16-input forward oracle on those
    values: MHA and GQA, both mask modes, a ragged length."""
    for (B, Hq, Hkv, N, D) in ((2, 4, 2, 37, 16), (1, 3, 3, 20, 8)):
        q8 = _codes(1700 + N, (B, Hq, N, D))
        k8 = _codes(1701 + N, (B, Hkv, N, D))
        v8 = _codes(1702 + N, (B, Hkv, N, D))
        dq, dk, dv = 2.0 ** -5, 2.0 ** -6, 2.0 ** -3

        def bits(c, s):
            x = s * torch_decode(c)
            b = f32_to_bf16_bits(x.astype(np.float32))
            assert np.array_equal((b.astype(np.uint32) << 16).view(np.float32), x)
            return b

        for causal in (False, True):
            o, lse = fref(q8, k8, v8, dq, dk, dv, causal, SCALE)
            eo, el = oracle.attn_ref(bits(q8, dq), bits(k8, dk), bits(v8, dv), causal, SCALE,
                                     n_threads=1)
            close(o, eo, tol=1e-13, what=f"O vs bf16 oracle causal={causal}")
            close(lse, el, tol=1e-13, what=f"LSE vs bf16 oracle causal={causal}")


def pin_torch_sdpa_general_descales(fref, dec):
    """Descales that are not powers of two (so the products are not exact in
    any narrow format): torch's fp64 SDPA on the decoded, scaled tensors, and
    scipy's logsumexp of the scaled scores; GQA with 3 query heads per K/V head."""
    B, Hq, Hkv, N, D = 1, 6, 2, 29, 32
    q8 = _codes(1800, (B, Hq, N, D), 0.0137)
    k8 = _codes(1801, (B, Hkv, N, D), 0.0291)
    v8 = _codes(1802, (B, Hkv, N, D), 0.77)
    dq, dk, dv = 0.0137, 0.0291, 0.77
    qt = torch.from_numpy(dq * torch_decode(q8))
    kt = torch.from_numpy(dk * torch_decode(k8)).repeat_interleave(Hq // Hkv, dim=1)
    vt = torch.from_numpy(dv * torch_decode(v8)).repeat_interleave(Hq // Hkv, dim=1)
    for causal in (False, True):
        o, lse = fref(q8, k8, v8, dq, dk, dv, causal, SCALE)
        eo = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=causal,
                                                              scale=SCALE).numpy()
        s = SCALE * torch.matmul(qt, kt.transpose(-1, -2)).numpy()
        if causal:
            s = np.where(np.tril(np.ones((N, N), bool)), s, -np.inf)
        close(o, eo, tol=1e-12, what=f"O vs torch SDPA causal={causal}")
        close(lse, scipy.special.logsumexp(s, axis=-1), tol=1e-12,
              what=f"LSE vs logsumexp causal={causal}")


def pin_rows_subset(fref, dec):
    """Sampled rows equal the same rows of the full result, bit for bit."""
    B, Hq, Hkv, N, D = 2, 4, 1, 23, 16
    q8, k8, v8 = (_codes(1900, (B, Hq, N, D)), _codes(1901, (B, Hkv, N, D)),
                  _codes(1902, (B, Hkv, N, D)))
    rows = np.array([0, 5, 22, 23, 91, 183, 100], np.int64)
    for causal in (False, True):
        o, lse, mag, rms = fref(q8, k8, v8, 0.3, 0.2, 1.1, causal, SCALE,
                                mags=(2.0 ** -4, 2.0 ** -16))
        so, sl, sm, sr = fref(q8, k8, v8, 0.3, 0.2, 1.1, causal, SCALE, rows=rows,
                              mags=(2.0 ** -4, 2.0 ** -16))
        assert np.array_equal(so, o.reshape(-1, D)[rows]) and np.array_equal(sl, lse.reshape(-1)[rows])
        assert np.array_equal(sm, mag.reshape(-1, D)[rows])
        assert np.array_equal(sr, rms.reshape(-1, D)[rows])


# ---------------------------------------------------------------- error scale
def pin_error_scale_closed_forms(fref, dec):
    """The error-scale sum (and its quadrature counterpart) in cases with closed
    forms:
    * every V row equal: O = that row and both are 0 (up to the rounding of O);
    * two keys with equal scores: weights 1/2 each, sum = w_rel * |v1 - v2| / 2,
      quadrature sum = w_rel * |v1 - v2| * sqrt(2) / 4;
    * two keys whose scores differ by 30 (w_rel = 0, floor 1e-6): the sum is
      (1e-6 |v1 - O| + e^-30 |v2 - O|) / (1 + e^-30), the quadrature sum
      sqrt((1e-6 |v1 - O|)^2 + (e^-30 |v2 - O|)^2) / (1 + e^-30).
    Causal row 0 sees one key: O = V[0] and both are 0."""
    D = 8
    one = 0x38
    # (a) constant V
    q8 = _codes(2000, (1, 1, 9, D))
    k8 = _codes(2001, (1, 1, 9, D))
    row = _codes(2002, (1, 1, 1, D))
    v8 = np.repeat(row, 9, axis=2)
    o, lse, mag, rms = fref(q8, k8, v8, 0.5, 0.25, 0.75, False, SCALE, mags=(2.0 ** -4, 2.0 ** -16))
    vrow = 0.75 * dec(row[0, 0, 0])
    close(o[0, 0], np.broadcast_to(vrow, (9, D)), tol=1e-15, what="constant V")
    assert np.all(mag <= 1e-15 * np.abs(vrow)), "constant V: error scale not zero"
    assert np.all(rms <= 1e-15 * np.abs(vrow)), "constant V: quadrature scale not zero"
    # (b) equal scores
    k8 = np.repeat(_codes(2003, (1, 1, 1, D)), 2, axis=2)
    v8 = _codes(2004, (1, 1, 2, D))
    q8 = _codes(2005, (1, 1, 2, D))
    o, lse, mag, rms = fref(q8, k8, v8, 1.0, 1.0, 1.0, False, SCALE, mags=(2.0 ** -4, 2.0 ** -16))
    v = dec(v8[0, 0])
    close(o[0, 0, 0], (v[0] + v[1]) / 2, tol=1e-15, what="equal scores: mean of V")
    close(mag[0, 0, 0], 2.0 ** -4 * np.abs(v[0] - v[1]) / 2, tol=1e-15, what="equal scores: error scale")
    close(rms[0, 0, 0], 2.0 ** -4 * np.abs(v[0] - v[1]) * math.sqrt(2) / 4, tol=1e-15,
          what="equal scores: quadrature scale")
    # (c) scores 30 apart: q = e_0, k1 = (a, 0, ...), k2 = (b, 0, ...)
    q8 = np.zeros((1, 1, 2, D), np.uint8)
    q8[..., 0] = one
    k8 = np.zeros((1, 1, 2, D), np.uint8)
    k8[0, 0, 0, 0] = 0x70   # 128
    k8[0, 0, 1, 0] = 0x38   # 1
    scale = 30.0 / 127.0
    o, lse, mag, rms = fref(q8, k8, v8, 1.0, 1.0, 1.0, False, scale, mags=(0.0, 1e-6))
    t = math.exp(-30.0)
    eo = (v[0] + t * v[1]) / (1 + t)
    close(o[0, 0, 0], eo, tol=1e-15, what="scores 30 apart: O")
    close(lse[0, 0, 0], 128 * scale + math.log1p(t), tol=1e-15, what="scores 30 apart: LSE")
    emag = (1e-6 * np.abs(v[0] - eo) + t * np.abs(v[1] - eo)) / (1 + t)
    close(mag[0, 0, 0], emag, tol=1e-12, what="scores 30 apart: error scale")
    erms = np.hypot(1e-6 * np.abs(v[0] - eo), t * np.abs(v[1] - eo)) / (1 + t)
    close(rms[0, 0, 0], erms, tol=1e-12, what="scores 30 apart: quadrature scale")
    # causal row 0
    q8, k8, v8 = _codes(2006, (1, 2, 5, D)), _codes(2007, (1, 2, 5, D)), _codes(2008, (1, 2, 5, D))
    o, lse, mag, rms = fref(q8, k8, v8, 0.5, 0.5, 0.5, True, SCALE, mags=(2.0 ** -4, 2.0 ** -16))
    close(o[0, :, 0], 0.5 * dec(v8[0, :, 0]), tol=1e-15, what="causal row 0")
    assert np.all(mag[0, :, 0] == 0.0), "causal row 0: error scale not zero"
    assert np.all(rms[0, :, 0] == 0.0), "causal row 0: quadrature scale not zero"


ALL_PINS = [pin_decode_matches_torch, pin_decode_format_values, pin_equals_bf16_oracle,
            pin_torch_sdpa_general_descales, pin_rows_subset, pin_error_scale_closed_forms]
