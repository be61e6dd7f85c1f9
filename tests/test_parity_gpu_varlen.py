"""GPU parity of the packed variable-length / sliding-window forward
(attn_fwd_varlen) against the fp64 oracle, element by element, at the
forward's bar (tests/parity.py).

Small packed batches are compared in full: sequence lengths from 1 to past
several query tiles, an empty sequence, MHA/GQA/MQA, both mask modes, windows
on one or both sides (including a window of 0 and windows wider than the
sequence).  The benchmark workloads run at their real sizes in the launch
configuration the benchmark times; sequences are independent, so rows of
sequences cut out of the packed batch are compared against the oracle run on
those sequences alone, plus finiteness of everything else.
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


def run_varlen(q, k, v, cu, causal, scale, window):
    import torch
    import scaled_dot_product_17_amd as sdpa
    cu_t = torch.from_numpy(np.ascontiguousarray(cu, np.int32)).cuda()
    lens = np.diff(cu)
    o, lse = sdpa.fwd_varlen(to_gpu(q), to_gpu(k), to_gpu(v), cu_t, int(lens.max()), causal=causal,
                             scale=scale, window=window)
    torch.cuda.synchronize()
    return bf16_to_np(o), lse.cpu().numpy()


def packed(seed, Hq, Hkv, lens):
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    total = int(cu[-1])
    return (synth.normal_bf16(seed, (Hq, total, 128)), synth.normal_bf16(seed + 1, (Hkv, total, 128)),
            synth.normal_bf16(seed + 2, (Hkv, total, 128)), cu)


CASES = [
    ((4, 4, [300]), (-1, -1)),
    ((4, 2, [1, 17, 256, 0, 513, 40]), (-1, -1)),
    ((8, 1, [700, 33, 1000]), (-1, -1)),
    ((4, 2, [600, 257]), (128, 128)),
    ((4, 4, [900, 31]), (64, -1)),
    ((2, 2, [520, 3]), (0, 0)),
    ((2, 1, [777]), (-1, 32)),
    ((4, 2, [1100, 64]), (300, 0)),
    ((2, 2, [400, 100]), (1, 1)),
    ((2, 2, [260]), (5000, 5000)),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "hq%d_hkv%d_n%d_w%d_%d" % (
    c[0][0], c[0][1], len(c[0][2]), c[1][0], c[1][1]))
def test_varlen_small_full(case, causal):
    (Hq, Hkv, lens), window = case
    say(f"[varlen small] {case} causal={causal}")
    q, k, v, cu = packed(14000 + sum(lens) + window[0], Hq, Hkv, lens)
    o, lse = run_varlen(q, k, v, cu, causal, SCALE, window)
    o_ref, lse_ref = oracle.attn_varlen_ref(q, k, v, cu, causal, SCALE, *window)
    m = parity.compare(o, lse, o_ref, lse_ref)
    parity.check(m, f"{case} causal={causal}")


@pytest.mark.parametrize("heads", [(16, 2), (32, 4)], ids=["16groups_sliced", "32groups_whole"])
@pytest.mark.parametrize("causal,window", [(False, (-1, -1)), (True, (-1, -1)), (True, (200, 0)),
                                           (False, (64, 64))])
def test_varlen_dealt_groups_full(causal, window, heads):
    """Sequences of unequal lengths are dealt to the 8 XCDs in groups of
    (sequence, head) pairs: with fewer than 32 groups each group is cut into 8
    slices, one per XCD, run row by row; with 32 or more, whole groups go to
    the XCDs in turn.  Eight sequences (the longest, 1000 tokens, has 8 tiles
    of 128 rows, so groups hold 8 pairs) of 16 query heads make 16 groups (the
    sliced form: every XCD holds a slice of every group), of 32 query heads 32
    groups (the whole-group form, four rounds over the XCDs).  Every row is
    compared with the oracle, and the outputs start as NaN bytes, so every
    element must be written."""
    import torch
    import scaled_dot_product_17_amd as sdpa
    lens = [1000, 40, 300, 7, 650, 129, 2, 900]
    Hq, Hkv = heads
    n_qtiles = -(-max(lens) // 128)
    pairs = len(lens) * Hq
    group = min(pairs, -(-64 // n_qtiles))
    assert max(lens) * len(lens) * 4 > sum(lens) * 5            # unequal: dealt order
    assert -(-pairs // group) == Hq                             # 16: sliced, 32: whole groups
    say(f"[varlen dealt] heads={heads} causal={causal} window={window}")
    q, k, v, cu = packed(14900 + Hq, Hq, Hkv, lens)
    total = int(cu[-1])
    out = torch.full((Hq, total, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse_t = torch.full((Hq, total), float("nan"), dtype=torch.float32, device="cuda")
    o, lse = sdpa.fwd_varlen(to_gpu(q), to_gpu(k), to_gpu(v), torch.from_numpy(cu).cuda(),
                             max(lens), causal=causal, scale=SCALE, window=window, out=out, lse=lse_t)
    torch.cuda.synchronize()
    # the oracle per K/V head (its query heads), on host threads
    from concurrent.futures import ThreadPoolExecutor
    gs = Hq // Hkv
    with ThreadPoolExecutor(max_workers=Hkv) as ex:
        parts = list(ex.map(lambda g: oracle.attn_varlen_ref(q[g * gs:(g + 1) * gs], k[g:g + 1], v[g:g + 1], cu,
                                                             causal, SCALE, *window), range(Hkv)))
    o_ref = np.concatenate([x[0] for x in parts])
    lse_ref = np.concatenate([x[1] for x in parts])
    m = parity.compare(bf16_to_np(o), lse.cpu().numpy(), o_ref, lse_ref)
    say(f"  {m}")
    parity.check(m, f"dealt heads={heads} causal={causal} window={window}")


@pytest.mark.parametrize("scale", [-0.0625, 0.0, 0.5])
def test_varlen_other_scales(scale):
    q, k, v, cu = packed(14500, 4, 2, [333, 70])
    for causal, window in ((False, (50, 20)), (True, (-1, -1))):
        o, lse = run_varlen(q, k, v, cu, causal, scale, window)
        o_ref, lse_ref = oracle.attn_varlen_ref(q, k, v, cu, causal, scale, *window)
        parity.check(parity.compare(o, lse, o_ref, lse_ref), f"scale={scale}")


def test_varlen_matches_dense_for_one_sequence():
    """One sequence with no window is the dense forward (B = 1), bitwise."""
    import torch
    import scaled_dot_product_17_amd as sdpa
    q, k, v, cu = packed(14600, 8, 2, [1000])
    for causal in (False, True):
        o, lse = run_varlen(q, k, v, cu, causal, SCALE, (-1, -1))
        od, ld = sdpa.fwd(to_gpu(q)[None], to_gpu(k)[None], to_gpu(v)[None], causal=causal,
                          scale=SCALE)
        torch.cuda.synchronize()
        assert np.array_equal(o, bf16_to_np(od)[0]) and np.array_equal(lse, ld.cpu().numpy()[0])


def test_varlen_deterministic_and_errors():
    import torch
    import scaled_dot_product_17_amd as sdpa
    q, k, v, cu = packed(14700, 4, 4, [500, 300])
    a = run_varlen(q, k, v, cu, True, SCALE, (100, -1))
    b = run_varlen(q, k, v, cu, True, SCALE, (100, -1))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    cu_t = torch.from_numpy(cu).cuda()
    with pytest.raises(sdpa.AttnError) as e:
        sdpa.fwd_varlen(to_gpu(q), to_gpu(k), to_gpu(v), cu_t, 0)
    assert e.value.status == 2
    with pytest.raises(ValueError):
        sdpa.fwd_varlen(to_gpu(q), to_gpu(k), to_gpu(v), cu_t.long(), 500)


@pytest.mark.parametrize("name", list(synth.VARLEN_WORKLOADS))
def test_varlen_workload_sequences(name):
    import torch
    import scaled_dot_product_17_amd as sdpa
    w = synth.VARLEN_WORKLOADS[name]
    say(f"[varlen workload] {name}")
    q, k, v = w.generate()
    cu = w.cu_seqlens()
    lens = np.diff(cu)
    cu_t = torch.from_numpy(cu).cuda()
    o, lse = sdpa.fwd_varlen(to_gpu(q), to_gpu(k), to_gpu(v), cu_t, int(lens.max()),
                             causal=w.causal, scale=w.scale, window=(w.left, w.right))
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o.float()).all()) and bool(torch.isfinite(lse).all())
    of, lf = bf16_to_np(o), lse.cpu().numpy()
    # the shortest sequence and the first one; for the oracle's time, the first
    # two query heads (and their K/V heads) and at most 4096 rows: with a causal
    # mask the first rows of a sequence depend on no later token, and with a
    # right window only the last `right` rows of the cut see past it
    g = w.H_q // w.H_kv
    hq, hkv = 2, -(-2 // g)
    for s in sorted({int(np.argmin(lens)), 0}):
        a, b = int(cu[s]), int(cu[s + 1])
        b_cut = min(b, a + 4096)
        keep = b_cut - a
        if b_cut < b and not w.causal and w.right != 0:
            keep = b_cut - a - (w.right if w.right > 0 else b_cut - a)
        sub_cu = np.array([0, b_cut - a], np.int32)
        o_ref, lse_ref = oracle.attn_varlen_ref(q[:hq, a:b_cut], k[:hkv, a:b_cut], v[:hkv, a:b_cut],
                                                sub_cu, w.causal, w.scale, w.left, w.right)
        m = parity.compare(of[:hq, a:a + keep], lf[:hq, a:a + keep], o_ref[:, :keep],
                           lse_ref[:, :keep])
        say(f"  {name} sequence {s} rows [{a}, {a + keep}), heads 0-{hq - 1}: {m}")
        parity.check(m, f"{name} sequence {s}")


@pytest.mark.parametrize("causal", [False, True])
def test_equal_lengths_match_dense(causal):
    """A packed batch of sequences of one length (the longest within 1.25x the
    mean: the dense grid order, a few heads at a time) equals the dense kernel
    on the same batch bitwise, every row of every head: each row's arithmetic
    is the same, and a tile the order skipped or repeated would show."""
    import torch
    import scaled_dot_product_17_amd as sdpa
    S, L, Hq, Hkv = 6, 640, 4, 2
    q, k, v, cu = packed(14600, Hq, Hkv, [L] * S)
    o, lse = run_varlen(q, k, v, cu, causal, SCALE, (-1, -1))
    dense = lambda a, h: to_gpu(a).view(h, S, L, 128).transpose(0, 1).contiguous()
    od, ld = sdpa.fwd(dense(q, Hq), dense(k, Hkv), dense(v, Hkv), causal=causal, scale=SCALE)
    torch.cuda.synchronize()
    od = bf16_to_np(od).transpose(1, 0, 2, 3).reshape(Hq, S * L, 128)
    ld = ld.cpu().numpy().transpose(1, 0, 2).reshape(Hq, S * L)
    assert np.array_equal(o, od) and np.array_equal(lse, ld), "packed != dense"


def test_nearly_equal_lengths_full():
    """Lengths within 1.25x of the mean (dense grid order) with ragged tails and
    GQA, both masks: every row against the oracle."""
    q, k, v, cu = packed(14700, 8, 2, [500, 512, 480, 512, 431])
    for causal in (False, True):
        o, lse = run_varlen(q, k, v, cu, causal, SCALE, (-1, -1))
        o_ref, lse_ref = oracle.attn_varlen_ref(q, k, v, cu, causal, SCALE, -1, -1)
        m = parity.compare(o, lse, o_ref, lse_ref)
        say(f"  nearly equal lengths causal={causal}: {m}")
        parity.check(m, f"nearly equal lengths causal={causal}")


@pytest.mark.parametrize("causal,n,heads,window", [(False, 8192, 16, (-1, -1)), (True, 9000, 16, (-1, -1)),
                                                   (False, 5000, 16, (-1, -1)), (False, 4000, 16, (3999, 3999)),
                                                   (True, 4000, 32, (3999, -1))])
def test_four_and_eight_wave_workgroups_agree(causal, n, heads, window):
    """A single sequence through the packed entry point equals the dense kernel
    on grids where the dense path uses 8-wave workgroups (256 or more 256-row
    tiles, 512 or more causal), bitwise: each row's arithmetic does not depend
    on the workgroup size.  Without a window the packed launch takes 8-wave
    workgroups as well; with a window wide enough to change no row (N - 1
    keys) but narrower than 8192 keys it takes 4-wave ones."""
    import torch
    import scaled_dot_product_17_amd as sdpa
    q, k, v, cu = packed(14800 + n + heads, heads, 2, [n])
    o, lse = run_varlen(q, k, v, cu, causal, SCALE, window)
    od, ld = sdpa.fwd(to_gpu(q)[None], to_gpu(k)[None], to_gpu(v)[None], causal=causal, scale=SCALE)
    torch.cuda.synchronize()
    assert np.array_equal(o, bf16_to_np(od)[0]) and np.array_equal(lse, ld.cpu().numpy()[0])
