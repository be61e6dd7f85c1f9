"""GPU parity: the HIP kernel against the fp64 oracle, element by element.

Small shapes are compared in full (several query/key tiles, ragged tails,
MHA/GQA/MQA, both mask modes).  The full benchmark workloads run at their real
sizes in the same launch configuration the benchmark times, and are compared on
sampled rows the oracle computes one by one, plus properties that hold at any
size (finite outputs, determinism, GQA == repeated MHA, causal structure).
"""
import math
import sys
import zlib

import numpy as np
import pytest

import oracle
import synth
from tests import parity
from tests.gpu_util import run, to_gpu, bf16_to_np

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
    sdpa.load()   # raises if the library was not built


def inputs(B, Hq, Hkv, N, seed, mult=1.0):
    q = synth.normal_bf16(seed, (B, Hq, N, 128), mult)
    k = synth.normal_bf16(seed + 1, (B, Hkv, N, 128), mult)
    v = synth.normal_bf16(seed + 2, (B, Hkv, N, 128))
    return q, k, v


SMALL = [(1, 2, 2, 256), (2, 4, 2, 1), (1, 2, 1, 17), (1, 3, 3, 64), (1, 2, 2, 65),
         (2, 4, 4, 127), (1, 2, 2, 128), (1, 2, 2, 129), (1, 8, 2, 200), (2, 4, 1, 1000),
         (1, 2, 2, 777), (1, 16, 8, 384), (1, 4, 4, 1536)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "b%d_hq%d_hkv%d_n%d" % s)
def test_small_full(shape, causal):
    B, Hq, Hkv, N = shape
    say(f"[small] {shape} causal={causal}")
    q, k, v = inputs(B, Hq, Hkv, N, seed=7000 + N)
    o, lse = run(q, k, v, causal, SCALE)
    o_ref, lse_ref = oracle.attn_ref(q, k, v, causal, SCALE)
    m = parity.compare(o, lse, o_ref, lse_ref)
    parity.check(m, f"{shape} causal={causal}")


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_workload_sampled(name):
    import torch
    w = synth.WORKLOADS[name]
    say(f"[workload] {name}")
    q, k, v = w.generate()
    qg, kg, vg = to_gpu(q), to_gpu(k), to_gpu(v)
    import scaled_dot_product_17_amd as sdpa
    o, lse = sdpa.fwd(qg, kg, vg, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o.float()).all()) and bool(torch.isfinite(lse).all())
    rng = np.random.default_rng(zlib.crc32(name.encode()))   # stable across processes
    rows = parity.sample_rows(w.B, w.H_q, w.N, rng, per_head=24)
    o_ref, lse_ref = oracle.attn_ref(q, k, v, w.causal, w.scale, rows=rows)
    of = o.view(-1, 128)[torch.from_numpy(rows).cuda()]
    lf = lse.view(-1)[torch.from_numpy(rows).cuda()]
    m = parity.compare(bf16_to_np(of), lf.cpu().numpy(), o_ref, lse_ref)
    say(f"  {name}: {m}")
    parity.check(m, name)


@pytest.mark.parametrize("shape", [(1, 5, 5, 3000), (3, 5, 1, 1000), (1, 3, 3, 9000), (1, 3, 3, 44000)],
                         ids=lambda s: "b%d_hq%d_hkv%d_n%d" % s)
def test_causal_head_groups_full(shape):
    """Causal grids interleave the tiles of groups of heads (enough tiles to fill
    one XCD's workgroup slots).  Groups that would not split evenly over the 8
    XCDs (here: groups of 3 heads of 24 tiles leaving a short last one; 15
    heads in groups of 8; groups of 1 of 3 heads of 71 four-wave tiles, and
    of 172 eight-wave tiles) are full-sized instead (1, 5, 1 and 1 heads) and
    dealt to the XCDs in strided slices, over grids with padding workgroups
    for the last two shapes (216 for 213 tiles, 528 for 516).  Every row of
    every head must still be computed once and match the oracle: all rows, or
    for the longest shape the first and last row of every 128-row span."""
    B, Hq, Hkv, N = shape
    say(f"[causal groups] {shape}")
    q, k, v = inputs(B, Hq, Hkv, N, seed=7500 + N)
    o, lse = run(q, k, v, True, SCALE)
    if N <= 10000:
        o_ref, lse_ref = oracle.attn_ref(q, k, v, True, SCALE)
    else:
        starts = np.arange(0, N, 128)
        near = np.unique(np.concatenate([starts, np.minimum(starts + 127, N - 1)]))
        rows = np.concatenate([(b * Hq + h) * N + near for b in range(B) for h in range(Hq)]).astype(np.int64)
        o_ref, lse_ref = oracle.attn_ref(q, k, v, True, SCALE, rows=rows)
        o, lse = o.reshape(-1, o.shape[-1])[rows], lse.reshape(-1)[rows]
    m = parity.compare(o, lse, o_ref, lse_ref)
    parity.check(m, f"{shape} causal")


def test_deterministic():
    q, k, v = inputs(2, 8, 2, 2048, seed=9100)
    for causal in (False, True):
        a, la = run(q, k, v, causal, SCALE)
        b, lb = run(q, k, v, causal, SCALE)
        assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_gqa_equals_repeated_mha():
    B, Hq, Hkv, N = 2, 8, 2, 640
    q, k, v = inputs(B, Hq, Hkv, N, seed=9200)
    g = Hq // Hkv
    for causal in (False, True):
        a, la = run(q, k, v, causal, SCALE)
        b, lb = run(q, np.repeat(k, g, axis=1), np.repeat(v, g, axis=1), causal, SCALE)
        assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_causal_future_independence():
    B, H, N, i = 1, 4, 1000, 300
    q, k, v = inputs(B, H, H, N, seed=9300)
    k2, v2 = k.copy(), v.copy()
    k2[:, :, i + 1:] = synth.normal_bf16(9303, k2[:, :, i + 1:].shape, 3.0)
    v2[:, :, i + 1:] = synth.normal_bf16(9304, v2[:, :, i + 1:].shape)
    a, la = run(q, k, v, True, SCALE)
    b, lb = run(q, k2, v2, True, SCALE)
    assert np.array_equal(a[:, :, :i + 1], b[:, :, :i + 1])
    assert np.array_equal(la[:, :, :i + 1], lb[:, :, :i + 1])


def test_causal_row0_is_v0():
    B, Hq, Hkv, N = 2, 4, 2, 300
    q, k, v = inputs(B, Hq, Hkv, N, seed=9400, mult=3.0)
    o, lse = run(q, k, v, True, SCALE)
    vf = synth.bf16_bits_to_f32(v)
    kvh = np.arange(Hq) // (Hq // Hkv)
    assert np.array_equal(o[:, :, 0, :], vf[:, kvh, 0, :])
    qf, kf = synth.bf16_bits_to_f32(q).astype(np.float64), synth.bf16_bits_to_f32(k).astype(np.float64)
    s00 = SCALE * np.sum(qf[:, :, 0] * kf[:, kvh, 0], axis=-1)
    assert np.max(np.abs(lse[:, :, 0] - s00)) < 1e-3


@pytest.mark.parametrize("scale", [0.0, -SCALE, 0.5, 1e-3])
def test_other_scales(scale):
    B, Hq, Hkv, N = 1, 4, 2, 333
    q, k, v = inputs(B, Hq, Hkv, N, seed=9500)
    for causal in (False, True):
        o, lse = run(q, k, v, causal, scale)
        o_ref, lse_ref = oracle.attn_ref(q, k, v, causal, float(np.float32(scale)))
        parity.check(parity.compare(o, lse, o_ref, lse_ref), f"scale={scale} causal={causal}")


def test_zero_queries_uniform():
    B, H, N = 1, 2, 200
    q, k, v = inputs(B, H, H, N, seed=9600)
    q = np.zeros_like(q)
    o, lse = run(q, k, v, False, SCALE)
    vf = synth.bf16_bits_to_f32(v).astype(np.float64)
    assert np.max(np.abs(o - vf.mean(axis=2, keepdims=True))) < 1e-2
    assert np.max(np.abs(lse - math.log(N))) < 1e-5


def test_lse_optional():
    q, k, v = inputs(1, 2, 2, 300, seed=9700)
    a, _ = run(q, k, v, True, SCALE, lse=True)
    b, lb = run(q, k, v, True, SCALE, lse=False)
    assert lb is None and np.array_equal(a, b)


def test_errors_reported():
    import torch
    import scaled_dot_product_17_amd as sdpa
    q = torch.zeros(1, 2, 64, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(sdpa.AttnError) as e:
        sdpa.fwd(q, q, q)
    assert e.value.status == 4
    flat = torch.zeros(2 * 64 * 128 + 1, dtype=torch.bfloat16, device="cuda")
    mis = flat[1:].view(1, 2, 64, 128)
    ok = torch.zeros(1, 2, 64, 128, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(sdpa.AttnError) as e:
        sdpa.fwd(mis, ok, ok)
    assert e.value.status == 6
    with pytest.raises(sdpa.AttnError) as e:
        sdpa.fwd(ok, ok, ok, out=ok)
    assert e.value.status == 7


def test_long_sequence_sampled():
    """N = 262144 (causal GQA, one batch): byte offsets deep into a head panel
    and 8192 key blocks per row stream; sampled rows across the sequence,
    including the first and the last, against the oracle."""
    import torch
    import scaled_dot_product_17_amd as sdpa
    B, Hq, Hkv, N = 1, 2, 1, 262144
    say(f"[long sequence] N={N}")
    q = synth.normal_bf16(18000, (B, Hq, N, 128))
    k = synth.normal_bf16(18001, (B, Hkv, N, 128))
    v = synth.normal_bf16(18002, (B, Hkv, N, 128))
    o, lse = sdpa.fwd(to_gpu(q), to_gpu(k), to_gpu(v), causal=True, scale=SCALE)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(lse).all())
    rows = np.array([0, 1, 255, 256, N // 2 + 17, N - 257, N - 1, N, N + 4095, 2 * N - 1], np.int64)
    o_ref, lse_ref = oracle.attn_ref(q, k, v, True, SCALE, rows=rows)
    sel = torch.from_numpy(rows).cuda()
    m = parity.compare(bf16_to_np(o.view(-1, 128)[sel]), lse.view(-1)[sel].cpu().numpy(), o_ref, lse_ref)
    say(f"  N={N}: {m}")
    parity.check(m, f"N={N}")


def test_max_sequence_sampled():
    """N = 2^23 - 1, the longest head panel the kernels' 32-bit byte offsets
    allow (N * 256 bytes < 2^31; attn_fwd refuses 2^23), causal, one head.  Q,
    K and V repeat a seeded pattern of 65521 rows: a prime period, so an
    offset that wrapped at a power of two would read a different row.  Sampled
    rows, the last of which see every key, against the oracle."""
    import torch
    import scaled_dot_product_17_amd as sdpa
    N, P = (1 << 23) - 1, 65521
    say(f"[max sequence] N={N}")
    q = np.resize(synth.normal_bf16(18100, (P, 128)), (1, 1, N, 128))
    k = np.resize(synth.normal_bf16(18101, (P, 128)), (1, 1, N, 128))
    v = np.resize(synth.normal_bf16(18102, (P, 128)), (1, 1, N, 128))
    o, lse = sdpa.fwd(to_gpu(q), to_gpu(k), to_gpu(v), causal=True, scale=SCALE)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 31, 32, P + 5, N // 2 + 7, N - 257, N - 33, N - 2, N - 1], np.int64)
    sel = torch.from_numpy(rows).cuda()
    og = bf16_to_np(o.view(-1, 128)[sel])
    lg = lse.view(-1)[sel].cpu().numpy()
    del o, lse
    o_ref, lse_ref = oracle.attn_ref(q, k, v, True, SCALE, rows=rows)
    m = parity.compare(og, lg, o_ref, lse_ref)
    say(f"  N={N}: {m}")
    parity.check(m, f"N={N}")
