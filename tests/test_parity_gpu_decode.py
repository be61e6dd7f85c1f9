"""GPU parity of split-KV decode and of the log-sum-exp merge against the fp64
oracles, element by element.

Decode uses the forward's bar (tests/parity.py: max-abs 1e-2 on O with the
faithful-rounding exception, mean-abs 1e-3, LSE 1e-3).  Small shapes are
compared in full: several splits and ragged key tails, one and several
query-column blocks, MHA/GQA/MQA, both mask modes, other scales, explicit and
automatic split counts.  The benchmark workloads run at their real sizes in the
launch configuration the benchmark times and are compared in full too (the
oracle's cost is M*L*D per row).  The merge kernel is checked on random
partials, including empty parts, against the merge oracle.
"""
import math
import sys

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
    sdpa.load()


def inputs(B, Hq, Hkv, M, L, seed):
    return (synth.normal_bf16(seed, (B, Hq, M, 128)), synth.normal_bf16(seed + 1, (B, Hkv, L, 128)),
            synth.normal_bf16(seed + 2, (B, Hkv, L, 128)))


def run_decode(q, k, v, causal, scale, n_splits=0):
    import torch
    import scaled_dot_product_17_amd as sdpa
    o, lse = sdpa.decode(to_gpu(q), to_gpu(k), to_gpu(v), causal=causal, scale=scale,
                         n_splits=n_splits)
    torch.cuda.synchronize()
    return bf16_to_np(o), lse.cpu().numpy()


SMALL = [(1, 2, 2, 1, 1), (1, 4, 2, 1, 17), (2, 8, 2, 1, 1000), (1, 16, 1, 1, 4096),
         (1, 8, 2, 4, 333), (2, 4, 4, 16, 2048), (1, 32, 2, 3, 777), (1, 16, 16, 1, 100),
         (1, 8, 1, 5, 5), (2, 6, 3, 2, 63)]


@pytest.mark.parametrize("n_splits", [0, 1, 5])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "b%d_hq%d_hkv%d_m%d_l%d" % s)
def test_decode_small_full(shape, causal, n_splits):
    B, Hq, Hkv, M, L = shape
    say(f"[decode small] {shape} causal={causal} n_splits={n_splits}")
    q, k, v = inputs(B, Hq, Hkv, M, L, seed=13000 + L + M)
    o, lse = run_decode(q, k, v, causal, SCALE, n_splits)
    o_ref, lse_ref = oracle.attn_decode_ref(q, k, v, causal, SCALE)
    m = parity.compare(o, lse, o_ref, lse_ref)
    parity.check(m, f"{shape} causal={causal} splits={n_splits}")


@pytest.mark.parametrize("scale", [-0.0625, 0.0, 0.5])
def test_decode_other_scales(scale):
    q, k, v = inputs(1, 8, 2, 3, 500, seed=13500)
    for causal in (False, True):
        o, lse = run_decode(q, k, v, causal, scale, 4)
        o_ref, lse_ref = oracle.attn_decode_ref(q, k, v, causal, scale)
        parity.check(parity.compare(o, lse, o_ref, lse_ref), f"scale={scale} causal={causal}")


def test_decode_deterministic_and_split_count():
    """Bitwise reproducible for a fixed split count; every split count meets the bar."""
    q, k, v = inputs(2, 8, 2, 2, 3000, seed=13600)
    a = run_decode(q, k, v, True, SCALE, 9)
    b = run_decode(q, k, v, True, SCALE, 9)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    o_ref, lse_ref = oracle.attn_decode_ref(q, k, v, True, SCALE)
    for s in (1, 2, 9, 94, 1000):
        o, lse = run_decode(q, k, v, True, SCALE, s)
        parity.check(parity.compare(o, lse, o_ref, lse_ref), f"n_splits={s}")


def test_decode_workspace_reuse_and_errors():
    import torch
    import scaled_dot_product_17_amd as sdpa
    q, k, v = inputs(1, 4, 1, 2, 300, seed=13700)
    qg, kg, vg = to_gpu(q), to_gpu(k), to_gpu(v)
    need = sdpa.attn_decode_workspace_bytes(1, 4, 1, 2, 300, 128, 3)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")   # stale garbage
    o_ref, lse_ref = oracle.attn_decode_ref(q, k, v, False, SCALE)
    for _ in range(2):
        o, lse = sdpa.decode(qg, kg, vg, n_splits=3, workspace=ws)
        torch.cuda.synchronize()
        parity.check(parity.compare(bf16_to_np(o), lse.cpu().numpy(), o_ref, lse_ref), "reuse")
    with pytest.raises(sdpa.AttnError) as e:
        sdpa.decode(qg, kg, vg, n_splits=3, workspace=ws[: need - 4])
    assert e.value.status == 10
    with pytest.raises(sdpa.AttnError) as e:
        sdpa.decode(qg[:, :, :2].contiguous(), kg[:, :, :1].contiguous(), vg[:, :, :1].contiguous(),
                    causal=True)
    assert e.value.status == 2


def test_lse_merge_kernel():
    """Random fp32 partials (some rows with empty parts, one row all empty, parts
    far apart in LSE) against the merge oracle."""
    import torch
    import scaled_dot_product_17_amd as sdpa
    rng = np.random.default_rng(5)
    for rows, P in ((1, 1), (37, 3), (300, 64), (5, 300)):
        op = rng.standard_normal((rows, P, 128)).astype(np.float32)
        lp = (rng.standard_normal((rows, P)) * 8).astype(np.float32)
        if rows > 2:
            lp[1, : P // 2] = -np.inf
            op[1, : P // 2] = 0
            lp[2, :] = -np.inf
            op[2] = 0
            lp[0, 0] = 300.0
        o, lse = sdpa.lse_merge(torch.from_numpy(op).cuda(), torch.from_numpy(lp).cuda())
        torch.cuda.synchronize()
        o_ref, lse_ref = oracle.attn_lse_merge_ref(op.astype(np.float64), lp.astype(np.float64))
        og = bf16_to_np(o).astype(np.float64)
        lg = lse.cpu().numpy().astype(np.float64)
        # bf16 output rounding plus fp32 weights and sums
        tol = 2.0 ** -8 * np.abs(o_ref) + 1e-5 * np.abs(op).max(axis=1)
        assert np.all(np.abs(og - o_ref) <= tol), f"merge O rows={rows} P={P}"
        fin = np.isfinite(lse_ref)
        assert np.array_equal(np.isfinite(lg), fin), "empty rows must give -inf"
        assert np.all(np.abs(lg[fin] - lse_ref[fin]) <= 1e-5 * (1 + np.abs(lse_ref[fin])))
        assert np.all(og[~fin] == 0)


def test_lse_merge_nonfinite_parts():
    """A NaN LSE_p makes its row NaN, beside finite and beside empty parts (the
    merge oracle's IEEE reading); an empty part (LSE -inf, O 0) beside finite
    ones is left out; a row of empty parts is O = 0, LSE = -inf."""
    import torch
    import scaled_dot_product_17_amd as sdpa
    rng = np.random.default_rng(6)
    rows, P = 6, 5
    op = rng.standard_normal((rows, P, 128)).astype(np.float32)
    lp = (rng.standard_normal((rows, P)) * 4).astype(np.float32)
    lp[0, 2] = np.nan                      # NaN beside finite parts
    lp[1, :] = -np.inf; op[1] = 0; lp[1, 3] = np.nan   # NaN beside empty parts
    lp[2, :] = -np.inf; op[2] = 0          # all empty
    lp[3, 1:] = -np.inf; op[3, 1:] = 0     # one finite part, the rest empty
    lp[4, 0] = np.inf                      # +inf: exp(inf - inf) is NaN
    o, lse = sdpa.lse_merge(torch.from_numpy(op).cuda(), torch.from_numpy(lp).cuda())
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_lse_merge_ref(op.astype(np.float64), lp.astype(np.float64))
    og = bf16_to_np(o).astype(np.float64)
    lg = lse.cpu().numpy().astype(np.float64)
    for name, g, r in (("O", og, o_ref), ("LSE", lg, lse_ref)):
        for kind, f in (("NaN", np.isnan), ("+inf", np.isposinf), ("-inf", np.isneginf)):
            assert np.array_equal(f(g), f(r)), f"merge {name} {kind} pattern {f(g)} vs {f(r)}"
    assert np.isnan(lg[[0, 1, 4]]).all() and lg[2] == -np.inf and np.all(og[2] == 0)
    fin = np.isfinite(o_ref)
    assert np.all(np.abs(og[fin] - o_ref[fin]) <= 2.0 ** -8 * np.abs(o_ref[fin]) + 1e-5 * 4)


def test_decode_partial_then_merge():
    """attn_decode_partial's splits match the oracle over their key ranges, and
    merging them with attn_lse_merge reproduces attn_decode bitwise."""
    import torch
    import scaled_dot_product_17_amd as sdpa
    B, Hq, Hkv, M, L, S = 1, 8, 2, 2, 1000, 6
    q, k, v = inputs(B, Hq, Hkv, M, L, seed=13800)
    qg, kg, vg = to_gpu(q), to_gpu(k), to_gpu(v)
    rows = B * Hq * M
    op = torch.empty((rows, S, 128), dtype=torch.float32, device="cuda")
    lp = torch.empty((rows, S), dtype=torch.float32, device="cuda")
    sp = torch.cuda.current_stream().cuda_stream
    assert sdpa.attn_decode_partial(qg.data_ptr(), kg.data_ptr(), vg.data_ptr(), op.data_ptr(),
                                    lp.data_ptr(), B, Hq, Hkv, M, L, 128, False, SCALE, S, sp) == 0
    o_m, l_m = sdpa.lse_merge(op, lp)
    o_d, l_d = sdpa.decode(qg, kg, vg, scale=SCALE, n_splits=S)
    torch.cuda.synchronize()
    assert torch.equal(o_m.view(torch.int16), o_d.view(torch.int16).view(rows, 128))
    assert torch.equal(l_m, l_d.view(rows))
    nb = (L + 31) // 32
    opn, lpn = op.cpu().numpy(), lp.cpu().numpy()
    for s in range(S):
        lo, hi = 32 * (s * nb // S), min(L, 32 * ((s + 1) * nb // S))
        o_ref, lse_ref = oracle.attn_decode_ref(q, k[:, :, lo:hi], v[:, :, lo:hi], False, SCALE)
        m = parity.compare(opn[:, s], lpn[:, s], o_ref.reshape(rows, 128), lse_ref.reshape(rows))
        parity.check(m, f"split {s} keys [{lo}, {hi})")


@pytest.mark.parametrize("name", list(synth.DECODE_WORKLOADS))
def test_decode_workload_full(name):
    w = synth.DECODE_WORKLOADS[name]
    say(f"[decode workload] {name}")
    q, k, v = w.generate()
    o, lse = run_decode(q, k, v, w.causal, w.scale)
    o_ref, lse_ref = oracle.attn_decode_ref(q, k, v, w.causal, w.scale)
    m = parity.compare(o, lse, o_ref, lse_ref)
    say(f"  {name}: {m}")
    parity.check(m, name)
