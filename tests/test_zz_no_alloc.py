"""attn_decode_noalloc, the decode entry point for callers that cannot
allocate device memory, through the C ABI.

Two calls in a row on one GPU, the second with a smaller input, so it runs on
the scratch array the first call left its partial results in.  Each is checked
against attn_decode (the entry point with a caller-owned workspace) on the
same inputs and split count, bitwise (both run the same kernels), and against
the fp64 decode oracle with the forward's bar (tests/parity.py).  A call whose
partial results would not fit the array is refused with ATTN_ERR_SCRATCH and
writes nothing.
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


def both_entry_points(B, Hq, Hkv, M, L, causal, n_splits, seed):
    """(o, lse) of attn_decode and of attn_decode_noalloc on the same inputs."""
    import torch
    import scaled_dot_product_17_amd as sdpa
    q = synth.normal_bf16(seed, (B, Hq, M, 128))
    k = synth.normal_bf16(seed + 1, (B, Hkv, L, 128))
    v = synth.normal_bf16(seed + 2, (B, Hkv, L, 128))
    qg, kg, vg = to_gpu(q), to_gpu(k), to_gpu(v)
    need = sdpa.attn_decode_workspace_bytes(B, Hq, Hkv, M, L, 128, n_splits)
    assert 0 < need <= sdpa.DECODE_SCRATCH_BYTES
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    outs = []
    for noalloc in (False, True):
        o = torch.full((B, Hq, M, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((B, Hq, M), float("nan"), dtype=torch.float32, device="cuda")
        stream = torch.cuda.current_stream().cuda_stream
        if noalloc:
            st = sdpa.attn_decode_noalloc(qg.data_ptr(), kg.data_ptr(), vg.data_ptr(), o.data_ptr(),
                                          lse.data_ptr(), B, Hq, Hkv, M, L, 128, causal, SCALE,
                                          n_splits, stream)
        else:
            st = sdpa.attn_decode(qg.data_ptr(), kg.data_ptr(), vg.data_ptr(), o.data_ptr(),
                                  lse.data_ptr(), B, Hq, Hkv, M, L, 128, causal, SCALE, n_splits,
                                  ws.data_ptr(), need, stream)
        assert st == sdpa.ATTN_OK, sdpa.status_string(st)
        torch.cuda.synchronize()
        outs.append((o, lse))
    (o_ws, l_ws), (o_na, l_na) = outs
    assert torch.equal(o_ws.view(torch.int16), o_na.view(torch.int16))
    assert torch.equal(l_ws.view(torch.int32), l_na.view(torch.int32))
    o_ref, lse_ref = oracle.attn_decode_ref(q, k, v, causal, SCALE)
    m = parity.compare(bf16_to_np(o_na), l_na.cpu().numpy(), o_ref, lse_ref)
    parity.check(m, f"noalloc B={B} Hq={Hq} Hkv={Hkv} M={M} L={L} causal={causal}")


def test_noalloc_two_calls_second_smaller():
    # the decode benchmark's shape (64 splits: 4.2 MB of partial results), then a
    # smaller causal GQA call with a ragged key tail and an explicit split count
    say("[noalloc] call 1: B=8 H_q=16 H_kv=2 M=1 L=32768")
    both_entry_points(8, 16, 2, 1, 32768, False, 0, 9100)
    say("[noalloc] call 2: B=2 H_q=8 H_kv=1 M=4 L=3001 causal n_splits=5")
    both_entry_points(2, 8, 1, 4, 3001, True, 5, 9110)


def test_noalloc_refuses_what_does_not_fit():
    import torch
    import scaled_dot_product_17_amd as sdpa
    B, Hq, Hkv, M, L, S = 8, 16, 16, 16, 4096, 64
    assert sdpa.attn_decode_workspace_bytes(B, Hq, Hkv, M, L, 128, S) > sdpa.DECODE_SCRATCH_BYTES
    q = torch.zeros((B, Hq, M, 128), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((B, Hkv, L, 128), dtype=torch.bfloat16, device="cuda")
    o = torch.full_like(q, 7.0)
    st = sdpa.attn_decode_noalloc(q.data_ptr(), kv.data_ptr(), kv.data_ptr(), o.data_ptr(), 0,
                                  B, Hq, Hkv, M, L, 128, False, SCALE, S,
                                  torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 11 and sdpa.STATUS_NAMES[st] == "ATTN_ERR_SCRATCH"
    assert bool((o == 7.0).all())
