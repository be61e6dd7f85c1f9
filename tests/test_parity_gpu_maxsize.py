"""GPU parity at the largest sizes each entry point accepts.

Every kernel addresses a head panel (or a packed batch, or a K/V cache) with
32-bit byte offsets, so the limit is 2^31 bytes of 256-byte bf16 rows: 2^23 - 1
rows (the ABI tests check that 2^23 is refused); block-sparse has a lower one,
2048 key blocks.  Each test runs one entry point at its limit and checks the
rows (or keys) at the deepest offsets against the oracle.  Q, K, V and dO repeat a seeded pattern of 65521 rows: a
prime period, so an offset that wrapped at a power of two would read a
different row and change the result.
"""
import math
import sys
import time

import numpy as np
import pytest

import oracle
import synth
from tests import parity
from tests.gpu_util import bf16_to_np, to_gpu

pytestmark = pytest.mark.gpu

SCALE = float(np.float32(1 / math.sqrt(128)))
NMAX = (1 << 23) - 1
PERIOD = 65521


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import scaled_dot_product_17_amd as sdpa
    sdpa.load()


def pmap(fn, items):
    """fn over items on host threads (the oracle's C calls release the GIL)."""
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=max(1, len(items))) as ex:
        return list(ex.map(fn, items))


def tiled(seed, shape):
    """bf16 bits of `shape` [..., n, 128]: a seeded [PERIOD, 128] pattern repeated along n."""
    return np.resize(synth.normal_bf16(seed, (PERIOD, 128)), shape)


def tiled_e4m3(seed, shape, descale):
    return np.resize(synth.normal_e4m3(seed, (PERIOD, 128), descale), shape)


def test_decode_max_cache():
    """Split-KV decode against a cache of 2^23 - 1 keys (bottom-right causal)."""
    import torch
    import scaled_dot_product_17_amd as sdpa
    B, Hq, Hkv, M, L = 1, 2, 1, 2, NMAX
    say(f"[max decode] L={L}")
    q = synth.normal_bf16(26000, (B, Hq, M, 128))
    k = tiled(26001, (B, Hkv, L, 128))
    v = tiled(26002, (B, Hkv, L, 128))
    o, lse = sdpa.decode(to_gpu(q), to_gpu(k), to_gpu(v), causal=True, scale=SCALE)
    torch.cuda.synchronize()
    parts = pmap(lambda h: oracle.attn_decode_ref(q[:, h:h + 1], k, v, True, SCALE), range(Hq))
    o_ref = np.concatenate([x[0] for x in parts], axis=1)
    lse_ref = np.concatenate([x[1] for x in parts], axis=1)
    m = parity.compare(bf16_to_np(o).reshape(-1, 128), lse.cpu().numpy().reshape(-1),
                       o_ref.reshape(-1, 128), lse_ref.reshape(-1))
    say(f"  decode L={L}: {m}")
    parity.check(m, f"decode L={L}")


def test_fp8_max_sequence():
    """The FP8 forward over 2^23 - 1 tokens (causal, one head): the last rows,
    which see every key, against the FP8 oracle and its contract."""
    import torch
    import scaled_dot_product_17_amd as sdpa
    N = NMAX
    d = synth.FP8_DESCALE
    say(f"[max fp8] N={N}")
    q8 = tiled_e4m3(27000, (1, 1, N, 128), d)
    k8 = tiled_e4m3(27001, (1, 1, N, 128), d)
    v8 = tiled_e4m3(27002, (1, 1, N, 128), d)

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a, np.uint8)).cuda()

    o, lse = sdpa.fwd_fp8(up(q8), up(k8), up(v8), d, d, d, causal=True, scale=SCALE)
    torch.cuda.synchronize()
    rows = np.array([PERIOD + 3, N - 2, N - 1], np.int64)
    sel = torch.from_numpy(rows).cuda()
    og = bf16_to_np(o.view(-1, 128)[sel])
    lg = lse.view(-1)[sel].cpu().numpy()
    del o, lse
    qv = oracle.e4m3_decode(q8[0, 0, :PERIOD])
    kv = oracle.e4m3_decode(k8[0, 0, :PERIOD])
    serr = parity.fp8_score_err(qv, kv, SCALE, d, d)
    parts = pmap(lambda r: oracle.attn_fp8_ref(q8, k8, v8, d, d, d, True, SCALE, rows=np.array([r], np.int64),
                                               mags=parity.fp8_mags(serr)), list(rows))
    o_ref, lse_ref, mag, rms = (np.concatenate([x[i] for x in parts]) for i in range(4))
    m = parity.fp8_compare(og, lg, o_ref, lse_ref, mag, rms, serr, N)
    say(f"  fp8 N={N}: {m}")
    assert m["finite"] and m["n_over"] == 0 and m["lse_n_over"] == 0, m


def test_varlen_max_tokens():
    """A packed batch of 2^23 - 1 tokens (causal): a long first sequence and a
    short last one at the deepest offsets.  Rows of a sequence do not depend on
    its neighbours in the pack, so the short one is checked whole with the
    varlen oracle and the long one's last rows with the dense oracle on its
    slice."""
    import torch
    import scaled_dot_product_17_amd as sdpa
    total, short = NMAX, 1000
    lens = [total - short, short]
    cu = np.array([0, lens[0], total], np.int32)
    H = 1
    say(f"[max varlen] total={total} lens={lens}")
    q = tiled(28000, (H, total, 128))
    k = tiled(28001, (H, total, 128))
    v = tiled(28002, (H, total, 128))
    qg, kg, vg, cug = to_gpu(q), to_gpu(k), to_gpu(v), torch.from_numpy(cu).cuda()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    o, lse = sdpa.fwd_varlen(qg, kg, vg, cug, max(lens), causal=True, scale=SCALE)
    torch.cuda.synchronize()
    say(f"  kernel {time.perf_counter() - t0:.1f} s")
    del qg, kg, vg
    a = lens[0]
    og = bf16_to_np(o[:, a:])
    lg = lse[:, a:].cpu().numpy()
    rows = np.array([a - 257, a - 2, a - 1], np.int64)
    sel = torch.from_numpy(rows).cuda()
    og_long = bf16_to_np(o[0][sel])
    lg_long = lse[0][sel].cpu().numpy()
    del o, lse
    cu1 = np.array([0, short], np.int32)
    o_ref, lse_ref = oracle.attn_varlen_ref(q[:, a:], k[:, a:], v[:, a:], cu1, True, SCALE)
    m = parity.compare(og, lg, o_ref, lse_ref)
    say(f"  varlen last sequence: {m}")
    parity.check(m, "varlen last sequence")
    o_ref, lse_ref = oracle.attn_ref(q[None, :, :a], k[None, :, :a], v[None, :, :a], True, SCALE, rows=rows)
    m = parity.compare(og_long, lg_long, o_ref, lse_ref)
    say(f"  varlen first sequence, last rows: {m}")
    parity.check(m, "varlen first sequence")


def test_blocksparse_max_sequence():
    """Block-sparse at its own limit, 2048 key blocks (N = 262144; the union of
    a tile's lists is kept in LDS), causal with one mask per head: a local +
    global + random pattern, and the last two query blocks of each head (one
    tile) listing every key block, so the union fills to capacity.  Sampled
    rows, the deepest last, against the oracle."""
    import torch
    import scaled_dot_product_17_amd as sdpa
    N, Hq, Hkv = 2048 * 128, 2, 1
    nb = N // 128
    say(f"[max blocksparse] N={N} blocks={nb}")
    q = tiled(29000, (1, Hq, N, 128))
    k = tiled(29001, (1, Hkv, N, 128))
    v = tiled(29002, (1, Hkv, N, 128))
    lists = synth.sparse_pattern(29003, nb, Hq, 2, 1, 2, True)
    for h in range(Hq):
        for qb in (nb - 2, nb - 1):
            lists[h * nb + qb] = list(range(nb))
    ptr, idx = synth.lists_to_csr(lists)
    o, lse = sdpa.fwd_blocksparse(to_gpu(q), to_gpu(k), to_gpu(v), torch.from_numpy(ptr).cuda(),
                                  torch.from_numpy(idx).cuda(), causal=True, scale=SCALE)
    torch.cuda.synchronize()
    per_head = np.array([0, 127, 128, PERIOD + 9, N // 2 + 5, N - 257, N - 129, N - 2, N - 1])
    rows = np.concatenate([h * N + per_head for h in range(Hq)]).astype(np.int64)
    sel = torch.from_numpy(rows).cuda()
    og = bf16_to_np(o.view(-1, 128)[sel])
    lg = lse.view(-1)[sel].cpu().numpy()
    del o, lse
    o_ref, lse_ref = oracle.attn_blocksparse_ref(q, k, v, ptr, idx, 128, True, SCALE, rows=rows)
    m = parity.compare(og, lg, o_ref, lse_ref)
    say(f"  blocksparse N={N}: {m}")
    parity.check(m, f"blocksparse N={N}")


def test_bwd_max_sequence():
    """The backward over 2^23 - 1 tokens (causal, one head): dQ of the last
    rows (each sees every key) and dK, dV of the last keys (their rows are the
    last ones), against the oracle's row and key modes."""
    import torch
    import scaled_dot_product_17_amd as sdpa
    N = NMAX
    say(f"[max bwd] N={N}")
    q = tiled(30000, (1, 1, N, 128))
    k = tiled(30001, (1, 1, N, 128))
    v = tiled(30002, (1, 1, N, 128))
    do = tiled(30003, (1, 1, N, 128))
    qg, kg, vg, dog = to_gpu(q), to_gpu(k), to_gpu(v), to_gpu(do)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    o, lse = sdpa.fwd(qg, kg, vg, causal=True, scale=SCALE)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    dq, dk, dv, _ = sdpa.bwd(qg, kg, vg, o, lse, dog, causal=True, scale=SCALE)
    torch.cuda.synchronize()
    say(f"  forward {t1 - t0:.1f} s, backward {time.perf_counter() - t1:.1f} s")
    rows = np.array([N - 3, N - 1], np.int64)
    keys = np.array([N - 32, N - 17, N - 2, N - 1], np.int64)
    gq = bf16_to_np(dq.view(-1, 128)[torch.from_numpy(rows).cuda()])
    kidx = torch.from_numpy(keys).cuda()
    gk = bf16_to_np(dk.view(-1, 128)[kidx])
    gv = bf16_to_np(dv.view(-1, 128)[kidx])
    del qg, kg, vg, dog, o, lse, dq, dk, dv
    rq, mq = oracle.attn_bwd_ref(q, k, v, do, True, SCALE, rows=rows, mags=True)
    met = parity.bwd_compare(gq, rq, mq)
    say(f"  bwd dq rows: {met}")
    parity.bwd_check(met, "bwd dq")
    rk, rv, mk, mv = oracle.attn_bwd_ref(q, k, v, do, True, SCALE, keys=keys, mags=True)
    for nm, g, r, mg in (("dk", gk, rk, mk), ("dv", gv, rv, mv)):
        met = parity.bwd_compare(g, r, mg)
        say(f"  bwd {nm} keys: {met}")
        parity.bwd_check(met, f"bwd {nm}")
