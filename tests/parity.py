"""Parity metrics between the GPU output and the fp64 oracle.

The bar (max-abs <= 1e-2, mean-abs <= 1e-3 on O, max-abs <= 1e-3 on LSE, for
unit-normal inputs) is a stated tolerance for a bf16 output.  Where the exact
result itself is farther than 1e-2 from every bf16 value (|O| >= 4 has bf16
spacing 1/32), no bf16 output can meet the max-abs bound; such an element also
passes when it is one of the two bf16 values bracketing the exact result (a
faithful rounding).  Mean-abs and LSE bounds apply as stated.
"""
from __future__ import annotations

import numpy as np

from synth import bf16_bits_to_f32, f32_to_bf16_bits

MAX_ABS = 1e-2
MEAN_ABS = 1e-3
LSE_ABS = 1e-3


def _bf16_succ_pred(bits: np.ndarray, up: np.ndarray) -> np.ndarray:
    """bf16 neighbour of each finite value: toward +inf where ``up`` else toward -inf."""
    b = bits.astype(np.int32)
    neg = (b & 0x8000) != 0
    mag = b & 0x7FFF
    # moving away from zero increments the magnitude; toward zero decrements it
    away = np.where(neg, ~up, up)
    mag2 = np.where(away, mag + 1, np.where(mag == 0, 1, mag - 1))
    sign = np.where(mag == 0, np.where(up, 0, 0x8000), b & 0x8000)
    return (sign | mag2).astype(np.uint16)


def faithful(o: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """True where the float o equals one of the two bf16 values bracketing ref."""
    ref = np.asarray(ref, dtype=np.float64)
    b = f32_to_bf16_bits(ref.astype(np.float32))
    vb = bf16_bits_to_f32(b).astype(np.float64)
    other = bf16_bits_to_f32(_bf16_succ_pred(b, vb <= ref)).astype(np.float64)
    return (o == vb) | (o == other)


def compare(o_gpu, lse_gpu, o_ref, lse_ref):
    """Metrics dict for the GPU output (any float array) against the oracle (float64)."""
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    err = np.abs(o_gpu - o_ref)
    floor = np.abs(bf16_bits_to_f32(f32_to_bf16_bits(o_ref.astype(np.float32))) - o_ref)
    over = err > MAX_ABS
    unfaithful_over = over & ~faithful(o_gpu, o_ref) if over.any() else over
    m = {
        "max_abs": float(err.max()) if err.size else 0.0,
        "mean_abs": float(err.mean()) if err.size else 0.0,
        "floor_max_abs": float(floor.max()) if floor.size else 0.0,
        "floor_mean_abs": float(floor.mean()) if floor.size else 0.0,
        "n_over_max_abs": int(over.sum()),
        "n_over_not_faithful": int(unfaithful_over.sum()),
        "finite": bool(np.all(np.isfinite(o_gpu))),
    }
    if lse_gpu is not None:
        le = np.abs(np.asarray(lse_gpu, dtype=np.float64) - lse_ref)
        m["lse_max_abs"] = float(le.max()) if le.size else 0.0
        m["lse_finite"] = bool(np.all(np.isfinite(lse_gpu)))
    return m


def check(m, what=""):
    assert m["finite"], f"{what}: non-finite output {m}"
    assert m["n_over_not_faithful"] == 0, f"{what}: max-abs {m}"
    assert m["mean_abs"] <= MEAN_ABS, f"{what}: mean-abs {m}"
    if "lse_max_abs" in m:
        assert m["lse_finite"] and m["lse_max_abs"] <= LSE_ABS, f"{what}: LSE {m}"


def sample_rows(B, Hq, N, rng, per_head=24, tile=128, heads=None):
    """Flat row ids ((b*Hq + h)*N + i) covering the first and last rows, query-tile
    edges and random rows of each (b, h) (or of the given list of (b, h))."""
    pairs = heads if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]
    out = []
    edges = sorted({0, 1, N - 1, N - 2} | {min(N - 1, t + d) for t in range(tile, N, tile * 37)
                                           for d in (-1, 0)})
    for b, h in pairs:
        base = (b * Hq + h) * N
        rows = set(x for x in edges if 0 <= x < N)
        rows |= set(int(x) for x in rng.integers(0, N, per_head))
        out.extend(base + r for r in sorted(rows))
    return np.array(out, dtype=np.int64)


# ---------------------------------------------------------------- backward
# Each gradient element is a sum of products in which the kernel rounds one
# factor to bf16 (P for dV, dS for dK and dQ; nearest even, relative error at
# most U; for dK, dS is itself formed from the bf16 P), takes delta from a bf16
# O (error up to about 2U times a_i = sum_j P_ij sum_d |dO_id||V_jd|),
# accumulates in fp32 and rounds the result to bf16 once (relative error U).
# The oracle's error-scale sum ``mag`` is the same sum with every term replaced
# by its magnitude and |dP - delta| widened by a_i.  To first order the dS
# error is at most 2U P_ij (|dP_ij - delta_i| + a_i), so
# |g - ref| <= U |ref| + (2U + fp32 terms) * mag; KAPPA = 4 leaves a factor of
# about 2 for fp32 accumulation over up to 32K terms (worst case < U/2 * mag)
# and second-order terms; the 2^-24 relative floor covers fp32 round-off of
# elements whose every term is tiny.
U_BF16 = 2.0 ** -8
BWD_KAPPA = 4.0


def bwd_compare(g_gpu, g_ref, mag):
    """Metrics of one GPU gradient (any float array) against the oracle: the worst
    ratio of the error to its bound and the count of elements over it."""
    g = np.asarray(g_gpu, dtype=np.float64)
    err = np.abs(g - g_ref)
    floor = 2.0 ** -24 * (float(np.abs(g_ref).max()) if g_ref.size else 0.0)
    bound = U_BF16 * np.abs(g_ref) + BWD_KAPPA * U_BF16 * mag + floor
    ratio = err / np.where(bound > 0, bound, np.inf)
    return {
        "finite": bool(np.all(np.isfinite(g))),
        "max_abs": float(err.max()) if err.size else 0.0,
        "max_ratio": float(ratio.max()) if ratio.size else 0.0,
        "n_over": int((err > bound).sum()),
        "rel_fro": float(np.linalg.norm(g - g_ref) / max(np.linalg.norm(g_ref), 1e-300)),
    }


def bwd_check(m, what=""):
    assert m["finite"], f"{what}: non-finite gradient {m}"
    assert m["n_over"] == 0, f"{what}: error over U|g| + {BWD_KAPPA}U*mag {m}"


# ---------------------------------------------------------------------------
# FP8 (e4m3) forward accuracy contract.  It follows from the e4m3 format and
# one stated scaling rule, not from any kernel's choices:
#   * scaling rule: the softmax weights of a row are rounded to e4m3 in groups
#     of consecutive keys, each group multiplied first by the power of two that
#     puts its largest weight in (224, 448]: the top binade of e4m3 below its largest
#     finite value 448, i.e. the largest placement a power-of-two scale can
#     guarantee without overflow.  Power-of-two scales are exact, and the
#     matrix core takes them back exactly (per-lane E8M0 operand scales);
#   * e4m3 keeps 3 mantissa bits in its normal range (down to 2^-6), so a
#     rounded weight is within 2^-4 of itself, relatively; below 2^-6 the
#     spacing is 2^-9, so within 2^-10 absolutely, in scaled units, i.e.
#     within 2^-10 / 224 of its group's largest weight, and so of the row's
#     largest weight -> the oracle's error-scale sum with
#     (w_rel, w_floor) = (2^-4 + score_err, 2^-10 / 224); O is normalised by
#     the sum of the rounded weights, which is what that sum bounds to first
#     order;
#   * the FP8 matrix core accumulates the 64-term products with an error
#     below 2^-14 of sum |q_d k_d| <= 2^-14 ||q|| ||k|| (measured on gfx950 at
#     about 2^-18.6); times |scale dq dk| this is score_err (natural-log units),
#     which moves each weight by a relative score_err and the LSE by at most
#     score_err;
#   * bf16 output rounding (2^-9 relative) and fp32 arithmetic: 2^-8 |O| and a
#     factor 1.3 on the first-order sum (its second-order remainder, the
#     e4m3 weight sum's own rounding and the bf16 rounding of the error);
#   * LSE: fp32 sums of up to n_keys weights (n_keys * 2^-24 relative), the
#     score error and 2^-16 (1 + |LSE|) for exp2/log/fp32 products.
# That bound holds however the roundings line up; on diffuse rows it is far
# above the error independent roundings actually leave, so a second, typical-
# size check uses the oracle's quadrature sum rms (the standard deviation of
# the first-order change when every weight's rounding is independent with at
# most the stated size): the mean over all compared elements of
# |err| / (rms + 2^-9 |O| + 2^-40) must stay below FP8_MEAN_Z = 1 (zero-mean
# roundings give about 0.5 or less; a misplaced weight or key gives >> 1).
FP8_W_REL = 2.0 ** -4
FP8_W_FLOOR = 2.0 ** -10 / 224.0
FP8_KAPPA = 1.3
FP8_MFMA_REL = 2.0 ** -14
FP8_MEAN_Z = 1.0


def fp8_score_err(qvals, kvals, scale, dq, dk) -> float:
    """Bound on the error of one scaled score: qvals/kvals are decoded e4m3
    values (any shape with D last) of the rows involved."""
    qn = float(np.sqrt((np.asarray(qvals, np.float64) ** 2).sum(-1)).max()) if np.size(qvals) else 0.0
    kn = float(np.sqrt((np.asarray(kvals, np.float64) ** 2).sum(-1)).max()) if np.size(kvals) else 0.0
    return abs(scale * dq * dk) * FP8_MFMA_REL * qn * kn


def fp8_mags(score_err: float):
    """(w_rel, w_floor) to pass to the FP8 oracle's error-scale sum."""
    return (FP8_W_REL + score_err, FP8_W_FLOOR)


def fp8_compare(o_gpu, lse_gpu, o_ref, lse_ref, mag, rms, score_err, n_keys):
    o_gpu = np.asarray(o_gpu, np.float64)
    err = np.abs(o_gpu - o_ref)
    tol = 2.0 ** -8 * np.abs(o_ref) + FP8_KAPPA * mag
    ratio = err / np.maximum(tol, 1e-300)
    z = err / (rms + 2.0 ** -9 * np.abs(o_ref) + 2.0 ** -40)
    m = {"max_abs": float(err.max()) if err.size else 0.0,
         "mean_abs": float(err.mean()) if err.size else 0.0,
         "max_err_over_tol": float(ratio.max()) if err.size else 0.0,
         "mean_tol": float(tol.mean()) if tol.size else 0.0,
         "n_over": int((err > tol).sum()),
         "mean_z": float(z.mean()) if z.size else 0.0,
         "finite": bool(np.all(np.isfinite(o_gpu)))}
    if lse_gpu is not None:
        le = np.abs(np.asarray(lse_gpu, np.float64) - lse_ref)
        lt = 2.0 ** -16 * (1 + np.abs(lse_ref)) + score_err + n_keys * 2.0 ** -24
        m["lse_max_abs"] = float(le.max()) if le.size else 0.0
        m["lse_n_over"] = int((le > lt).sum())
    return m


def fp8_check(m, what=""):
    assert m["finite"], f"{what}: non-finite output"
    assert m["n_over"] == 0, f"{what}: {m['n_over']} outputs beyond the FP8 bound ({m})"
    assert m["mean_z"] <= FP8_MEAN_Z, f"{what}: typical error above the rounding scale ({m})"
    assert m.get("lse_n_over", 0) == 0, f"{what}: LSE beyond the FP8 bound ({m})"
