"""GPU parity of the block-sparse forward (attn_fwd_blocksparse) against the fp64
block-sparse oracle, element by element, at the forward's bar (tests/parity.py),
with rows that see no key checked for exactly O = 0 and LSE = -inf.

Small shapes are compared in full: lengths from 1 to several blocks with ragged
tails, MHA/GQA/MQA, one mask for all heads and one per head, both mask modes,
empty lists, diagonal-only lists, random lists with duplicate and out-of-range
entries.  Every block listed reproduces the dense kernel bitwise.  The benchmark
workloads run at their real sizes in the launch configuration the benchmark
times, compared on sampled rows.
"""
import math
import sys

import numpy as np
import pytest

import oracle
import synth
from tests import parity
from tests.gpu_util import bf16_to_np, poison_lds, to_gpu

pytestmark = pytest.mark.gpu

SCALE = float(np.float32(1 / math.sqrt(128)))
BLK = 128


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import scaled_dot_product_17_amd as sdpa
    sdpa.load()


def i32_gpu(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def run_bs(q, k, v, lists, causal, scale):
    import torch
    import scaled_dot_product_17_amd as sdpa
    ptr, idx = synth.lists_to_csr(lists)
    o, lse = sdpa.fwd_blocksparse(to_gpu(q), to_gpu(k), to_gpu(v), i32_gpu(ptr), i32_gpu(idx),
                                  causal=causal, scale=scale)
    torch.cuda.synchronize()
    return bf16_to_np(o), lse.cpu().numpy()


def check(o, lse, o_ref, lse_ref, what):
    empty = np.isneginf(lse_ref)
    assert np.all(o[empty] == 0.0) and np.all(np.isneginf(lse[empty])), f"{what}: empty rows"
    ok = ~empty
    if ok.any():
        m = parity.compare(o[ok], lse[ok], o_ref[ok], lse_ref[ok])
        parity.check(m, what)


def inputs(seed, B, Hq, Hkv, N):
    return (synth.normal_bf16(seed, (B, Hq, N, 128)), synth.normal_bf16(seed + 1, (B, Hkv, N, 128)),
            synth.normal_bf16(seed + 2, (B, Hkv, N, 128)))


def random_lists(seed, n_lists, nb, extra_junk=False):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n_lists):
        ls = sorted(set(rng.integers(0, nb, rng.integers(0, nb + 1)).tolist()))
        if extra_junk and ls:
            ls = ls + [ls[0], -3, nb + 5]      # a duplicate and two out-of-range entries
        out.append(ls)
    return out


SMALL = [(1, 2, 2, 1), (1, 2, 2, 100), (1, 4, 2, 128), (1, 4, 1, 300), (2, 4, 4, 513),
         (1, 8, 2, 1000)]


@pytest.mark.parametrize("per_head", [False, True])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "b%d_hq%d_hkv%d_n%d" % s)
def test_blocksparse_small_random(shape, causal, per_head):
    B, Hq, Hkv, N = shape
    nb = -(-N // BLK)
    say(f"[blocksparse small] {shape} causal={causal} per_head={per_head}")
    q, k, v = inputs(17000 + N, B, Hq, Hkv, N)
    lists = random_lists(N + 3 * per_head + causal, (Hq if per_head else 1) * nb, nb,
                         extra_junk=(N % 2 == 0))
    o, lse = run_bs(q, k, v, lists, causal, SCALE)
    ptr, idx = synth.lists_to_csr(lists)
    o_ref, lse_ref = oracle.attn_blocksparse_ref(q, k, v, ptr, idx, BLK, causal, SCALE)
    check(o, lse, o_ref, lse_ref, f"{shape} causal={causal} per_head={per_head}")


@pytest.mark.parametrize("causal", [False, True])
def test_blocksparse_full_lists_equal_dense_bitwise(causal):
    import torch
    import scaled_dot_product_17_amd as sdpa
    B, Hq, Hkv, N = 2, 4, 2, 700
    nb = -(-N // BLK)
    q, k, v = inputs(17500, B, Hq, Hkv, N)
    o, lse = run_bs(q, k, v, [list(range(nb))] * nb, causal, SCALE)
    od, ld = sdpa.fwd(to_gpu(q), to_gpu(k), to_gpu(v), causal=causal, scale=SCALE)
    torch.cuda.synchronize()
    assert np.array_equal(o, bf16_to_np(od)) and np.array_equal(lse, ld.cpu().numpy())


def test_blocksparse_structured_lists():
    """Diagonal-only lists, empty lists for some query blocks, a causal list of
    blocks after the diagonal only (rows that see nothing), other scales."""
    B, Hq, Hkv, N = 1, 4, 4, 640
    nb = N // BLK
    q, k, v = inputs(17600, B, Hq, Hkv, N)
    cases = [([[qb] for qb in range(nb)], SCALE),
             ([[], [0, 1], [], [3], [0, 4]], 0.5),
             ([[1, 2], [3], [3, 4], [], [4]], -0.0625),
             ([[0, 2, 4]] * nb, 0.0)]
    for lists, scale in cases:
        ptr, idx = synth.lists_to_csr(lists)
        for causal in (False, True):
            o, lse = run_bs(q, k, v, lists, causal, scale)
            o_ref, lse_ref = oracle.attn_blocksparse_ref(q, k, v, ptr, idx, BLK, causal, scale)
            check(o, lse, o_ref, lse_ref, f"lists={lists} scale={scale} causal={causal}")


def test_blocksparse_deterministic_and_errors():
    import torch
    import scaled_dot_product_17_amd as sdpa
    q, k, v = inputs(17700, 1, 2, 2, 400)
    lists = random_lists(5, 4, 4)
    a = run_bs(q, k, v, lists, True, SCALE)
    b = run_bs(q, k, v, lists, True, SCALE)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    ptr, idx = synth.lists_to_csr(lists)
    with pytest.raises(ValueError):           # 3 offsets for 4 query blocks
        sdpa.fwd_blocksparse(to_gpu(q), to_gpu(k), to_gpu(v), i32_gpu(ptr[:3]), i32_gpu(idx))
    # offsets past the index array are clamped: no fault, rows see what is listed
    bad_ptr = ptr.copy()
    bad_ptr[-1] = 10 ** 6
    o, lse = sdpa.fwd_blocksparse(to_gpu(q), to_gpu(k), to_gpu(v), i32_gpu(bad_ptr), i32_gpu(idx))
    torch.cuda.synchronize()
    assert o.shape == (1, 2, 400, 128)


@pytest.mark.parametrize("name", list(synth.SPARSE_WORKLOADS))
def test_blocksparse_workload_sampled(name):
    w = synth.SPARSE_WORKLOADS[name]
    say(f"[blocksparse workload] {name}")
    q, k, v = w.generate()
    lists = w.lists()
    o, lse = run_bs(q, k, v, lists, w.causal, w.scale)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    rng = np.random.default_rng(w.seed_base)
    total = w.B * w.H_q * w.N
    rows = [0, w.N - 1, total - 1, total - w.N]
    for t0 in range(0, w.N, 256):                      # first and last row of every tile, head 0
        rows += [t0, min(t0 + 255, w.N - 1)]
    rows = np.unique(np.concatenate([np.array(rows), rng.integers(0, total, 256)])).astype(np.int64)
    ptr, idx = w.csr()
    o_ref, lse_ref = oracle.attn_blocksparse_ref(q, k, v, ptr, idx, w.block, w.causal, w.scale,
                                                 rows=rows)
    m = parity.compare(o.reshape(-1, 128)[rows], lse.reshape(-1)[rows], o_ref, lse_ref)
    say(f"  {name}: {m}")
    parity.check(m, name)


@pytest.mark.parametrize("causal", [False, True])
def test_stale_lds_is_never_read(causal):
    """Launches whose LDS rings are not cleared first (block-sparse with N a
    multiple of 128, dense with N a multiple of 32) read only ring slots their
    own copies filled: after the LDS has been filled with NaN rows by other
    launches, they reproduce their results bitwise."""
    import torch
    import scaled_dot_product_17_amd as sdpa
    B, Hq, Hkv, N = 2, 8, 2, 1024
    nb = N // BLK
    q, k, v = inputs(17800, B, Hq, Hkv, N)
    lists = random_lists(17803, nb, nb)
    lists[1] = []                                   # a query block with no key
    lists[2] = [nb - 1]                              # only the last block (causal: nothing)
    ptr, idx = synth.lists_to_csr(lists)
    qg, kg, vg = to_gpu(q), to_gpu(k), to_gpu(v)

    def both():
        o1, l1 = sdpa.fwd_blocksparse(qg, kg, vg, i32_gpu(ptr), i32_gpu(idx), causal=causal, scale=SCALE)
        o2, l2 = sdpa.fwd(qg, kg, vg, causal=causal, scale=SCALE)
        torch.cuda.synchronize()
        return [bf16_to_np(o1), l1.cpu().numpy(), bf16_to_np(o2), l2.cpu().numpy()]

    first = both()
    poison_lds()
    after = both()
    for a, b in zip(first, after):
        assert np.array_equal(a, b, equal_nan=True)
    assert np.all(np.isfinite(after[0])) and np.all(np.isfinite(after[2]))
    o_ref, lse_ref = oracle.attn_blocksparse_ref(q, k, v, ptr, idx, BLK, causal, SCALE)
    check(after[0], after[1], o_ref, lse_ref, f"block-sparse after stale LDS, causal={causal}")
