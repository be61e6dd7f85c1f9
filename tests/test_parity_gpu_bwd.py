"""GPU parity of the backward pass: dQ, dK, dV from the HIP kernels against the
fp64 backward oracle, element by element.

The gradients come from the whole path a caller runs (the HIP forward's O and
LSE feed the HIP backward).  Each element must satisfy
|g - ref| <= U |ref| + KAPPA U mag (tests/parity.py derives the bound from the
kernel's arithmetic; ``mag`` is the oracle's error-scale sum).  Small shapes are
compared in full (several tiles of both kernels, ragged tails, MHA/GQA/MQA,
both mask modes, other scales).  The benchmark workloads run at their real
sizes in the launch configuration the benchmark times and are compared on
sampled dQ rows and sampled dK/dV key rows that the oracle computes on their
own, plus the column sum of dV, which holds at any size.
"""
import math
import sys
import zlib

import numpy as np
import pytest

import oracle
import synth
from tests import parity
from tests.gpu_util import bf16_to_np, to_gpu

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


def inputs(B, Hq, Hkv, N, seed):
    q = synth.normal_bf16(seed, (B, Hq, N, 128))
    k = synth.normal_bf16(seed + 1, (B, Hkv, N, 128))
    v = synth.normal_bf16(seed + 2, (B, Hkv, N, 128))
    do = synth.normal_bf16(seed + 3, (B, Hq, N, 128))
    return q, k, v, do


def run_bwd(q, k, v, do, causal, scale, o=None, lse=None, n_splits=0, workspace=None):
    """HIP forward (unless o, lse are given) then HIP backward (n_splits: parts of
    the dK/dV step, <= 0 the library's choice); numpy results."""
    import torch
    import scaled_dot_product_17_amd as sdpa
    qg, kg, vg, dog = to_gpu(q), to_gpu(k), to_gpu(v), to_gpu(do)
    if o is None:
        og, lg = sdpa.fwd(qg, kg, vg, causal=causal, scale=scale)
    else:
        og, lg = to_gpu(o), torch.from_numpy(np.ascontiguousarray(lse, np.float32)).cuda()
    dq, dk, dv, delta = sdpa.bwd(qg, kg, vg, og, lg, dog, causal=causal, scale=scale,
                                 n_splits=n_splits, workspace=workspace)
    torch.cuda.synchronize()
    return {"dq": bf16_to_np(dq), "dk": bf16_to_np(dk), "dv": bf16_to_np(dv),
            "delta": delta.cpu().numpy()}


def check_all(res, ref, what):
    dq, dk, dv, mq, mk, mv = ref
    for name, r, m in (("dq", dq, mq), ("dk", dk, mk), ("dv", dv, mv)):
        met = parity.bwd_compare(res[name], r, m)
        say(f"  {what} {name}: {met}")
        parity.bwd_check(met, f"{what} {name}")


SMALL = [(1, 2, 2, 256), (2, 4, 2, 1), (1, 2, 1, 17), (1, 3, 3, 64), (1, 2, 2, 65),
         (1, 2, 2, 129), (1, 8, 2, 200), (2, 4, 1, 1000), (1, 2, 2, 777), (1, 16, 8, 384),
         (1, 4, 4, 1536)]


@pytest.mark.parametrize("splits", [0, 1], ids=["auto_parts", "one_part"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "b%d_hq%d_hkv%d_n%d" % s)
def test_bwd_small_full(shape, causal, splits):
    """Both dK/dV forms: the library's choice (these small grids split every
    group of more than one query head) and one part (attn_bwd)."""
    B, Hq, Hkv, N = shape
    say(f"[bwd small] {shape} causal={causal} n_splits={splits}")
    q, k, v, do = inputs(B, Hq, Hkv, N, seed=11000 + N)
    res = run_bwd(q, k, v, do, causal, SCALE, n_splits=splits)
    ref = oracle.attn_bwd_ref(q, k, v, do, causal, SCALE, mags=True)
    check_all(res, ref, f"{shape} causal={causal} n_splits={splits}")


def test_bwd_split_parts():
    """attn_bwd_ws with 2, 4 and 8 parts of a 16-head group (GQA 16:2, ragged
    N): every part count meets the bound, dQ and delta equal the one-part
    result bitwise (the dQ kernel does not change), each part count is
    reproducible bitwise, and the workspace's old contents do not matter."""
    import torch
    import scaled_dot_product_17_amd as sdpa
    B, Hq, Hkv, N = 1, 16, 2, 1000
    q, k, v, do = inputs(B, Hq, Hkv, N, seed=13100)
    for causal in (False, True):
        ref = oracle.attn_bwd_ref(q, k, v, do, causal, SCALE, mags=True)
        one = run_bwd(q, k, v, do, causal, SCALE, n_splits=1)
        for ns in (2, 4, 8):
            assert sdpa.attn_bwd_splits(B, Hq, Hkv, N, 128, causal, ns) == ns
            need = sdpa.attn_bwd_workspace_bytes(B, Hq, Hkv, N, 128, causal, ns)
            assert need == ns * 2 * B * Hkv * N * 128 * 4
            ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")   # NaN bytes
            say(f"[bwd parts] causal={causal} n_splits={ns}")
            a = run_bwd(q, k, v, do, causal, SCALE, n_splits=ns, workspace=ws)
            b = run_bwd(q, k, v, do, causal, SCALE, n_splits=ns)
            check_all(a, ref, f"causal={causal} n_splits={ns}")
            for name in a:
                assert np.array_equal(a[name], b[name]), f"{name} differs between runs"
            for name in ("dq", "delta"):
                assert np.array_equal(a[name], one[name]), f"{name} depends on the dK/dV parts"


@pytest.mark.parametrize("scale", [-0.0625, 0.0, 0.5])
def _kgroup(B, Hkv, N, ns):
    """The causal dK/dV grid's interleave of (batch, K/V head, part) units, as
    attn_bwd_ws sets it: enough 128-key tiles to fill one XCD's 32 workgroup
    slots, at most all units."""
    n_ktiles = -(-N // 128)
    return min(B * Hkv * ns, -(-32 // n_ktiles))


def test_bwd_split_mqa_full():
    """The dK/dV split path of the long-context causal MQA workload (B=1,
    H_q=16, H_kv=1, N=32768: 8 parts of 2 query heads, one unit per causal
    interleave group) at N=4096, where the oracle computes every gradient:
    the same part count, heads per part and interleave, on peaky inputs
    (Q, K scaled by 3 as in that workload), compared element by element."""
    import scaled_dot_product_17_amd as sdpa
    B, Hq, Hkv, N_big, N = 1, 16, 1, 32768, 4096
    ns = sdpa.attn_bwd_splits(B, Hq, Hkv, N_big, 128, True, 0)
    assert ns == 8
    assert sdpa.attn_bwd_splits(B, Hq, Hkv, N, 128, True, ns) == ns
    assert _kgroup(B, Hkv, N_big, ns) == _kgroup(B, Hkv, N, ns) == 1
    q = synth.normal_bf16(13500, (B, Hq, N, 128), 3.0)
    k = synth.normal_bf16(13501, (B, Hkv, N, 128), 3.0)
    v = synth.normal_bf16(13502, (B, Hkv, N, 128))
    do = synth.normal_bf16(13503, (B, Hq, N, 128))
    say(f"[bwd mqa split] N={N} n_splits={ns}")
    res = run_bwd(q, k, v, do, True, SCALE, n_splits=ns)
    ref = oracle.attn_bwd_ref(q, k, v, do, True, SCALE, mags=True)
    check_all(res, ref, f"causal MQA N={N} n_splits={ns}")


@pytest.mark.parametrize("scale", [-0.0625, 0.0, 0.5])
def test_bwd_other_scales(scale):
    say(f"[bwd scale] {scale}")
    q, k, v, do = inputs(1, 4, 2, 300, seed=12000)
    for causal in (False, True):
        res = run_bwd(q, k, v, do, causal, scale)
        ref = oracle.attn_bwd_ref(q, k, v, do, causal, scale, mags=True)
        check_all(res, ref, f"scale={scale} causal={causal}")


def test_bwd_delta_from_given_o():
    """O and LSE taken from the oracle (rounded to bf16 / fp32) instead of the
    HIP forward: delta must be the fp32 row sum dO . O of that O, and the
    gradients must still meet the bound."""
    say("[bwd delta]")
    B, Hq, Hkv, N = 1, 4, 2, 333
    q, k, v, do = inputs(B, Hq, Hkv, N, seed=12500)
    for causal in (False, True):
        o_ref, lse_ref = oracle.attn_ref(q, k, v, causal, SCALE)
        o_bits = synth.f32_to_bf16_bits(o_ref.astype(np.float32))
        res = run_bwd(q, k, v, do, causal, SCALE, o=o_bits, lse=lse_ref.astype(np.float32))
        terms = synth.bf16_bits_to_f32(do).astype(np.float64) * \
            synth.bf16_bits_to_f32(o_bits).astype(np.float64)
        exact = terms.sum(axis=-1)
        tol = 2.0 ** -17 * np.abs(terms).sum(axis=-1) + 1e-30
        assert np.all(np.abs(res["delta"] - exact) <= tol), "delta != dO . O"
        check_all(res, oracle.attn_bwd_ref(q, k, v, do, causal, SCALE, mags=True),
                  f"given O causal={causal}")


def test_bwd_deterministic():
    q, k, v, do = inputs(2, 8, 2, 1024, seed=12600)
    for causal in (False, True):
        a = run_bwd(q, k, v, do, causal, SCALE)
        b = run_bwd(q, k, v, do, causal, SCALE)
        for name in a:
            assert np.array_equal(a[name], b[name]), f"{name} differs between runs"


def test_bwd_gqa_dq_equals_repeated_mha():
    """dQ of GQA equals dQ of MHA with K/V repeated per group (same arithmetic)."""
    B, Hq, Hkv, N = 1, 8, 2, 400
    q, k, v, do = inputs(B, Hq, Hkv, N, seed=12700)
    g = Hq // Hkv
    for causal in (False, True):
        a = run_bwd(q, k, v, do, causal, SCALE)
        b = run_bwd(q, np.repeat(k, g, axis=1), np.repeat(v, g, axis=1), do, causal, SCALE)
        assert np.array_equal(a["dq"], b["dq"])


def _panel_keys(B, Hkv, N, panels, rng, per_panel=16):
    out = []
    for b, kv in panels:
        js = {0, 1, N - 1, N - 2, 127, 128} | set(rng.integers(0, N, per_panel).tolist())
        out += [(b * Hkv + kv) * N + j for j in sorted(j for j in js if 0 <= j < N)]
    return np.array(out, np.int64)


BWD_WORKLOADS = ["mha_noncausal_b2_h16_n16384", "mha_causal_b2_h16_n16384",
                 "gqa_b8_hq16_hkv2_n2048", "mqa_causal_peaky_b1_hq16_n32768"]


@pytest.mark.parametrize("name", BWD_WORKLOADS)
def test_bwd_workload_sampled(name):
    import torch
    import scaled_dot_product_17_amd as sdpa
    w = synth.WORKLOADS[name]
    say(f"[bwd workload] {name}")
    q, k, v = w.generate()
    do = synth.normal_bf16(w.seed_base + 3, q.shape)
    qg, kg, vg, dog = to_gpu(q), to_gpu(k), to_gpu(v), to_gpu(do)
    o, lse = sdpa.fwd(qg, kg, vg, causal=w.causal, scale=w.scale)
    dq, dk, dv, _ = sdpa.bwd(qg, kg, vg, o, lse, dog, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    for t in (dq, dk, dv):
        assert bool(torch.isfinite(t.float()).all())
    rng = np.random.default_rng(zlib.crc32(name.encode()))   # stable across processes

    # dQ on sampled rows
    rows = parity.sample_rows(w.B, w.H_q, w.N, rng, per_head=8)
    rq, mq = oracle.attn_bwd_ref(q, k, v, do, w.causal, w.scale, rows=rows, mags=True)
    gq = bf16_to_np(dq.view(-1, 128)[torch.from_numpy(rows).cuda()])
    met = parity.bwd_compare(gq, rq, mq)
    say(f"  {name} dq rows: {met}")
    parity.bwd_check(met, f"{name} dq")

    # dK, dV on sampled keys of one or two K/V panels.  The oracle needs every
    # row of those panels' query heads that sees a sampled key: all rows, or
    # with the causal mask the rows from the smallest sampled key on.  Where
    # all rows of a group would take too long (the 16-head causal MQA panel at
    # 32768 tokens: 16 * 32768 rows), the keys come from the panel's last
    # 1024, i.e. its last 8 key tiles (the same dK/dV parts and sum; the
    # split grid at a smaller size is compared in full by
    # test_bwd_split_mqa_full).
    group_rows = (w.H_q // w.H_kv) * w.N * w.N
    panels = [(0, 0)] if group_rows > 2 ** 28 or w.B * w.H_kv == 1 else \
        [(0, 0), (w.B - 1, w.H_kv - 1)]
    if group_rows <= 2 ** 30:
        keys = _panel_keys(w.B, w.H_kv, w.N, panels, rng)
    else:
        assert w.causal, "a non-causal group this large has no cheap key sample"
        lo = w.N - 1024
        js = {lo, lo + 1, lo + 127, lo + 128, w.N - 129, w.N - 128, w.N - 2, w.N - 1} | \
            set(int(x) for x in rng.integers(lo, w.N, 40))
        keys = np.array(sorted(js), np.int64)   # panel (0, 0)
    say(f"  {name}: oracle dK/dV for {len(keys)} keys")
    rk, rv, mk, mv = oracle.attn_bwd_ref(q, k, v, do, w.causal, w.scale, keys=keys, mags=True)
    kidx = torch.from_numpy(keys).cuda()
    for nm, g, r, m in (("dk", dk, rk, mk), ("dv", dv, rv, mv)):
        met = parity.bwd_compare(bf16_to_np(g.view(-1, 128)[kidx]), r, m)
        say(f"  {name} {nm} keys: {met}")
        parity.bwd_check(met, f"{name} {nm}")

    # every row of P sums to one: sum_j dV_j = sum of dO over the group's rows,
    # within U (sum_j |dV_j| + sum_i |dO_i|) (the rounding of P and of dV)
    g = w.H_q // w.H_kv
    dv64 = dv.double().view(w.B, w.H_kv, w.N, 128)
    do64 = dog.double().view(w.B, w.H_kv, g * w.N, 128)
    lhs = dv64.sum(dim=2)
    rhs = do64.sum(dim=2)
    tol = 1.25 * parity.U_BF16 * (dv64.abs().sum(dim=2) + do64.abs().sum(dim=2))
    over = int(((lhs - rhs).abs() > tol).sum())
    say(f"  {name} sum dV: max |diff| {float((lhs - rhs).abs().max()):.3e}, over {over}")
    assert over == 0, "sum_j dV_j != sum_i dO_i"


def test_bwd_split_calls_match():
    """attn_bwd_dq then attn_bwd_dkdv (raw C-ABI calls) give attn_bwd's outputs bitwise."""
    import torch
    import scaled_dot_product_17_amd as sdpa
    B, Hq, Hkv, N = 1, 4, 2, 700
    q, k, v, do = inputs(B, Hq, Hkv, N, seed=12800)
    qg, kg, vg, dog = to_gpu(q), to_gpu(k), to_gpu(v), to_gpu(do)
    for causal in (False, True):
        o, lse = sdpa.fwd(qg, kg, vg, causal=causal, scale=SCALE)
        dq, dk, dv, delta = sdpa.bwd(qg, kg, vg, o, lse, dog, causal=causal, scale=SCALE,
                                     n_splits=1)
        dq2, dk2, dv2 = torch.empty_like(qg), torch.empty_like(kg), torch.empty_like(vg)
        delta2 = torch.empty_like(lse)
        sp = torch.cuda.current_stream().cuda_stream
        a = (B, Hq, Hkv, N, 128, causal, SCALE, sp)
        assert sdpa.attn_bwd_dq(qg.data_ptr(), kg.data_ptr(), vg.data_ptr(), o.data_ptr(),
                                dog.data_ptr(), lse.data_ptr(), dq2.data_ptr(),
                                delta2.data_ptr(), *a) == 0
        assert sdpa.attn_bwd_dkdv(qg.data_ptr(), kg.data_ptr(), vg.data_ptr(), dog.data_ptr(),
                                  lse.data_ptr(), delta2.data_ptr(), dk2.data_ptr(),
                                  dv2.data_ptr(), *a) == 0
        torch.cuda.synchronize()
        for x, y in ((dq, dq2), (dk, dk2), (dv, dv2), (delta, delta2)):
            assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x,
                               y.view(torch.int16) if y.dtype == torch.bfloat16 else y)


def test_bwd_errors_reported():
    import torch
    import scaled_dot_product_17_amd as sdpa
    q, k, v, do = inputs(1, 4, 2, 64, seed=12900)
    qg, kg, vg, dog = to_gpu(q), to_gpu(k), to_gpu(v), to_gpu(do)
    o, lse = sdpa.fwd(qg, kg, vg)
    with pytest.raises(sdpa.AttnError) as e:
        sdpa.bwd(qg, kg, vg, o, lse, dog, scale=float("nan"))
    assert e.value.status == 5
    with pytest.raises(ValueError):
        sdpa.bwd(qg, kg, vg, o, lse[:, :, :10].contiguous(), dog)
    bad = torch.empty(1, 4, 64, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(sdpa.AttnError) as e:
        sdpa.bwd(bad, kg[..., :64].contiguous(), vg[..., :64].contiguous(), bad, lse, bad)
    assert e.value.status == 4
    # a split call with too small a workspace (2 parts of the 4:2 group)
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(sdpa.AttnError) as e:
        sdpa.bwd(qg, kg, vg, o, lse, dog, n_splits=2, workspace=small)
    assert e.value.status == 10
