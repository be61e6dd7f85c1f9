"""GPU parity of the FP8 (e4m3) forward (attn_fwd_fp8) against the fp64 FP8
oracle, element by element, at the derived FP8 bound (tests/parity.py:
2^-8 |O| + 1.3 x the oracle's error-scale sum for e4m3 weights on every
element, the mean error within the quadrature rounding scale, LSE within the
score error plus fp32 rounding).

Small shapes are compared in full: lengths from 1 to several key blocks with
ragged tails, one and several query tiles, MHA/GQA/MQA, both mask modes, other
scales and descales (negative, zero, non-powers of two), peaky rows that move
the softmax reference, and constant scores.  The FP8 workloads run at their
real sizes in the launch configuration the benchmark times, compared on
sampled rows (first and last rows of query tiles and seeded random rows).
"""
import math
import sys

import numpy as np
import pytest

import oracle
import synth
from tests import parity
from tests.gpu_util import bf16_to_np

pytestmark = pytest.mark.gpu

SCALE = float(np.float32(1 / math.sqrt(128)))


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import scaled_dot_product_17_amd as sdpa
    sdpa.load()


def u8_gpu(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def run_fp8(q8, k8, v8, dq, dk, dv, causal, scale):
    import torch
    import scaled_dot_product_17_amd as sdpa
    o, lse = sdpa.fwd_fp8(u8_gpu(q8), u8_gpu(k8), u8_gpu(v8), dq, dk, dv, causal=causal,
                          scale=scale)
    torch.cuda.synchronize()
    return bf16_to_np(o), lse.cpu().numpy()


def decoded(codes):
    return oracle.e4m3_decode(codes)


def check_rows(o, lse, q8, k8, v8, dq, dk, dv, causal, scale, rows=None, what=""):
    """Compare GPU rows (all, or flat row ids) with the oracle at the FP8 bound."""
    B, Hq, N, D = q8.shape
    qv = decoded(q8.reshape(-1, D) if rows is None else q8.reshape(-1, D)[rows])
    serr = parity.fp8_score_err(qv, decoded(k8), scale, dq, dk)
    o_ref, lse_ref, mag, rms = oracle.attn_fp8_ref(q8, k8, v8, dq, dk, dv, causal, scale,
                                                   rows=rows, mags=parity.fp8_mags(serr))
    if rows is None:
        og, lg = o, lse
    else:
        og, lg = o.reshape(-1, D)[rows], lse.reshape(-1)[rows]
    m = parity.fp8_compare(og, lg, o_ref, lse_ref, mag, rms, serr, N)
    say(f"  {what}: {m}")
    parity.fp8_check(m, what)
    return m


def codes(seed, shape, descale=synth.FP8_DESCALE):
    return synth.normal_e4m3(seed, shape, descale)


SMALL = [(1, 2, 2, 1), (1, 2, 2, 17), (1, 2, 2, 64), (1, 4, 2, 65), (2, 4, 2, 127),
         (1, 8, 1, 300), (1, 2, 2, 513), (2, 4, 4, 256), (1, 6, 3, 200)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "b%d_hq%d_hkv%d_n%d" % s)
def test_fp8_small_full(shape, causal):
    B, Hq, Hkv, N = shape
    say(f"[fp8 small] {shape} causal={causal}")
    q8 = codes(15000 + N, (B, Hq, N, 128))
    k8 = codes(15001 + N, (B, Hkv, N, 128))
    v8 = codes(15002 + N, (B, Hkv, N, 128))
    d = synth.FP8_DESCALE
    o, lse = run_fp8(q8, k8, v8, d, d, d, causal, SCALE)
    check_rows(o, lse, q8, k8, v8, d, d, d, causal, SCALE, what=f"{shape} causal={causal}")


def test_fp8_causal_head_groups_full():
    """Causal FP8 grids interleave the tiles of groups of heads (8 heads of 8
    tiles here) and the last group is short (7 heads): every row of every head
    must still be computed once and meet the bound."""
    B, Hq, Hkv, N = 3, 5, 1, 1000
    say(f"[fp8 causal groups] {(B, Hq, Hkv, N)}")
    q8 = codes(15500, (B, Hq, N, 128))
    k8 = codes(15501, (B, Hkv, N, 128))
    v8 = codes(15502, (B, Hkv, N, 128))
    d = synth.FP8_DESCALE
    o, lse = run_fp8(q8, k8, v8, d, d, d, True, SCALE)
    check_rows(o, lse, q8, k8, v8, d, d, d, True, SCALE, what="causal head groups")


@pytest.mark.parametrize("scale,dq,dk,dv", [
    (SCALE, 0.0137, 0.0291, 0.77), (-0.0625, 0.02, 0.02, 1.0), (0.0, 0.02, 0.02, 0.5),
    (SCALE, 0.013, 0.014, -2.5), (0.5, 0.013, 0.013, 0.013)])
def test_fp8_scales_and_descales(scale, dq, dk, dv):
    B, Hq, Hkv, N = 1, 4, 2, 333
    q8, k8, v8 = codes(15500, (B, Hq, N, 128)), codes(15501, (B, Hkv, N, 128)), \
        codes(15502, (B, Hkv, N, 128))
    for causal in (False, True):
        o, lse = run_fp8(q8, k8, v8, dq, dk, dv, causal, scale)
        check_rows(o, lse, q8, k8, v8, dq, dk, dv, causal, scale,
                   what=f"scale={scale} d=({dq},{dk},{dv}) causal={causal}")


def test_fp8_peaky_rows_move_the_reference():
    """Scores with a spread of tens of nats: later keys exceed the first block's
    maximum by far, so the reference moves (rare path) many times per row."""
    B, Hq, Hkv, N = 1, 4, 1, 700
    q8, k8 = codes(15600, (B, Hq, N, 128)), codes(15601, (B, Hkv, N, 128))
    # keys whose magnitude grows along the sequence: each block outscores the last
    ramp = np.linspace(0.2, 1.0, N)[None, None, :, None]
    kv = decoded(k8) * ramp
    k8 = synth.f64_to_e4m3(kv)
    v8 = codes(15602, (B, Hkv, N, 128))
    for causal in (False, True):
        o, lse = run_fp8(q8, k8, v8, 0.05, 0.05, 0.1, causal, 0.3)
        check_rows(o, lse, q8, k8, v8, 0.05, 0.05, 0.1, causal, 0.3, what=f"peaky causal={causal}")


def test_fp8_constant_scores():
    """Identical keys: every weight is the reference weight (their sum passes the
    check threshold in every block) and O is the mean of V."""
    B, Hq, Hkv, N = 1, 2, 1, 1000
    q8 = codes(15700, (B, Hq, N, 128))
    k8 = np.repeat(codes(15701, (B, Hkv, 1, 128)), N, axis=2)
    v8 = codes(15702, (B, Hkv, N, 128))
    for causal in (False, True):
        o, lse = run_fp8(q8, k8, v8, 0.02, 0.02, 0.5, causal, SCALE)
        check_rows(o, lse, q8, k8, v8, 0.02, 0.02, 0.5, causal, SCALE,
                   what=f"constant scores causal={causal}")


def test_fp8_deterministic_and_float8_dtype():
    import torch
    import scaled_dot_product_17_amd as sdpa
    q8, k8, v8 = codes(15800, (2, 4, 600, 128)), codes(15801, (2, 2, 600, 128)), \
        codes(15802, (2, 2, 600, 128))
    a = run_fp8(q8, k8, v8, 0.02, 0.02, 0.5, True, SCALE)
    b = run_fp8(q8, k8, v8, 0.02, 0.02, 0.5, True, SCALE)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    f8 = [u8_gpu(x).view(torch.float8_e4m3fn) for x in (q8, k8, v8)]
    o, lse = sdpa.fwd_fp8(*f8, 0.02, 0.02, 0.5, causal=True, scale=SCALE)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_to_np(o), a[0]) and np.array_equal(lse.cpu().numpy(), a[1])
    with pytest.raises(sdpa.AttnError) as e:
        sdpa.fwd_fp8(*f8, float("nan"), 1.0, 1.0)
    assert e.value.status == 5


def sample_rows(B, Hq, N, n, seed):
    """First and last rows of every 256-row query tile of head 0 and the last
    head, plus n seeded random rows."""
    rng = np.random.default_rng(seed)
    picks = []
    for b, h in ((0, 0), (B - 1, Hq - 1)):
        for t0 in range(0, N, 256):
            for i in (t0, min(t0 + 255, N - 1)):
                picks.append((b * Hq + h) * N + i)
    picks.extend(rng.integers(0, B * Hq * N, n).tolist())
    return np.unique(np.array(picks, np.int64))


@pytest.mark.parametrize("name", list(synth.FP8_WORKLOADS))
def test_fp8_workload_sampled(name):
    w = synth.FP8_WORKLOADS[name]
    say(f"[fp8 workload] {name}")
    q8, k8, v8 = w.generate()
    o, lse = run_fp8(q8, k8, v8, w.descale_q, w.descale_k, w.descale_v, w.causal, w.scale)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    n = 64 if w.N >= 16384 else 256
    rows = sample_rows(w.B, w.H_q, w.N, n, 16000 + w.seed_base) if w.N > 256 else None
    check_rows(o, lse, q8, k8, v8, w.descale_q, w.descale_k, w.descale_v, w.causal, w.scale,
               rows=rows, what=name)
