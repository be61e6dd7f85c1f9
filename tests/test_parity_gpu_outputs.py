"""Every entry point writes every element of its outputs.

Caller-provided output buffers are filled with NaN bytes (0xFF) first. Each
call must then give bitwise the results of a call into fresh buffers. That
includes rows past a ragged tail, rows that see no key (block-sparse:
O = 0, LSE = -inf), the LSE and delta vectors, and every head of a GQA group.
Parity with the oracle is covered by each path's own tests.
"""
import math
import sys

import numpy as np
import pytest

import synth
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


def nan_like(t):
    """A buffer of t's shape and dtype holding 0xFF bytes (NaN in bf16 and fp32)."""
    import torch
    b = torch.empty_like(t)
    b.view(torch.uint8).fill_(0xFF)
    return b


def to_np(t):
    import torch
    return bf16_to_np(t) if t.dtype == torch.bfloat16 else t.cpu().numpy()


def same(fresh, filled, what):
    import torch
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(fresh, filled)):
        x, y = to_np(a), to_np(b)
        assert np.array_equal(x, y), f"{what}: output {i} differs when its buffer held NaN bytes"
        assert not np.isnan(y).any(), f"{what}: output {i} kept NaN bytes"


def bf16(seed, shape):
    return to_gpu(synth.normal_bf16(seed, shape))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 4, 2, 1000), (2, 2, 2, 64), (1, 8, 1, 4097)],
                         ids=lambda s: "b%d_hq%d_hkv%d_n%d" % s)
def test_fwd_outputs_overwritten(shape, causal):
    import scaled_dot_product_17_amd as sdpa
    B, Hq, Hkv, N = shape
    say(f"[outputs] fwd {shape} causal={causal}")
    q, k, v = bf16(18300, (B, Hq, N, 128)), bf16(18301, (B, Hkv, N, 128)), bf16(18302, (B, Hkv, N, 128))
    fresh = sdpa.fwd(q, k, v, causal=causal, scale=SCALE)
    o, lse = nan_like(fresh[0]), nan_like(fresh[1])
    filled = sdpa.fwd(q, k, v, causal=causal, scale=SCALE, out=o, lse=lse)
    same(fresh, filled, f"fwd {shape} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_outputs_overwritten(causal):
    import torch
    import scaled_dot_product_17_amd as sdpa
    B, Hq, Hkv, N = 1, 4, 2, 1000
    say(f"[outputs] fp8 causal={causal}")
    d = synth.FP8_DESCALE
    q8, k8, v8 = (torch.from_numpy(synth.normal_e4m3(18400 + i, (B, h, N, 128), d)).cuda()
                  for i, h in enumerate((Hq, Hkv, Hkv)))
    fresh = sdpa.fwd_fp8(q8, k8, v8, d, d, d, causal=causal, scale=SCALE)
    o, lse = nan_like(fresh[0]), nan_like(fresh[1])
    filled = sdpa.fwd_fp8(q8, k8, v8, d, d, d, causal=causal, scale=SCALE, out=o, lse=lse)
    same(fresh, filled, f"fp8 causal={causal}")


@pytest.mark.parametrize("causal,window", [(True, (-1, -1)), (False, (100, 50))])
def test_varlen_outputs_overwritten(causal, window):
    import torch
    import scaled_dot_product_17_amd as sdpa
    lens = [1, 300, 17, 1000, 129]
    total = sum(lens)
    say(f"[outputs] varlen causal={causal} window={window}")
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)).cuda()
    q, k, v = bf16(18500, (4, total, 128)), bf16(18501, (2, total, 128)), bf16(18502, (2, total, 128))
    fresh = sdpa.fwd_varlen(q, k, v, cu, max(lens), causal=causal, scale=SCALE, window=window)
    o, lse = nan_like(fresh[0]), nan_like(fresh[1])
    filled = sdpa.fwd_varlen(q, k, v, cu, max(lens), causal=causal, scale=SCALE, window=window,
                             out=o, lse=lse)
    same(fresh, filled, f"varlen causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_blocksparse_outputs_overwritten(causal):
    import torch
    import scaled_dot_product_17_amd as sdpa
    B, Hq, Hkv, N = 1, 4, 2, 700
    nb = -(-N // 128)
    say(f"[outputs] blocksparse causal={causal}")
    lists = [[0, 2], [], [5], [1, 3], [4], [0, 5]]   # an empty list; a list after the diagonal
    assert len(lists) == nb
    ptr, idx = synth.lists_to_csr(lists)
    pg, ig = torch.from_numpy(ptr).cuda(), torch.from_numpy(idx).cuda()
    q, k, v = bf16(18600, (B, Hq, N, 128)), bf16(18601, (B, Hkv, N, 128)), bf16(18602, (B, Hkv, N, 128))
    fresh = sdpa.fwd_blocksparse(q, k, v, pg, ig, causal=causal, scale=SCALE)
    o, lse = nan_like(fresh[0]), nan_like(fresh[1])
    filled = sdpa.fwd_blocksparse(q, k, v, pg, ig, causal=causal, scale=SCALE, out=o, lse=lse)
    same(fresh, filled, f"blocksparse causal={causal}")


@pytest.mark.parametrize("n_splits", [1, 0])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_outputs_overwritten(causal, n_splits):
    import scaled_dot_product_17_amd as sdpa
    B, Hq, Hkv, N = 1, 4, 1, 1000
    say(f"[outputs] bwd causal={causal} n_splits={n_splits}")
    q, k, v = bf16(18700, (B, Hq, N, 128)), bf16(18701, (B, Hkv, N, 128)), bf16(18702, (B, Hkv, N, 128))
    do = bf16(18703, (B, Hq, N, 128))
    o, lse = sdpa.fwd(q, k, v, causal=causal, scale=SCALE)
    fresh = sdpa.bwd(q, k, v, o, lse, do, causal=causal, scale=SCALE, n_splits=n_splits)
    bufs = [nan_like(t) for t in fresh]
    filled = sdpa.bwd(q, k, v, o, lse, do, causal=causal, scale=SCALE, n_splits=n_splits,
                      dq=bufs[0], dk=bufs[1], dv=bufs[2], delta=bufs[3])
    same(fresh, filled, f"bwd causal={causal} n_splits={n_splits}")


@pytest.mark.parametrize("M,L,causal", [(1, 1000, False), (5, 333, True)])
def test_decode_outputs_overwritten(M, L, causal):
    import scaled_dot_product_17_amd as sdpa
    B, Hq, Hkv = 2, 8, 2
    say(f"[outputs] decode M={M} L={L} causal={causal}")
    q, k, v = bf16(18800, (B, Hq, M, 128)), bf16(18801, (B, Hkv, L, 128)), bf16(18802, (B, Hkv, L, 128))
    fresh = sdpa.decode(q, k, v, causal=causal, scale=SCALE)
    o, lse = nan_like(fresh[0]), nan_like(fresh[1])
    filled = sdpa.decode(q, k, v, causal=causal, scale=SCALE, out=o, lse=lse)
    same(fresh, filled, f"decode M={M} L={L} causal={causal}")
