"""Stream ordering and concurrent callers.

The library enqueues every launch on the stream it is given, and the binding
passes torch's current stream. So a call made on a side stream runs after the
work queued before it on that stream, even while that stream is still busy.
The library keeps no state between calls, so two host threads driving two
streams at once get the results of sequential calls. Streams here use the
default priority.
"""
import math
import sys
import threading

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


def to_np(t):
    import torch
    return bf16_to_np(t) if t.dtype == torch.bfloat16 else t.cpu().numpy()


def bf16(seed, shape):
    return to_gpu(synth.normal_bf16(seed, shape))


def busy(n=3):
    """Queue some milliseconds of unrelated work on the current stream."""
    import torch
    a = torch.full((4096, 4096), 1.0 / 4096, device="cuda")
    for _ in range(n):
        a = a @ a


@pytest.mark.parametrize("op", ["fwd", "bwd", "decode"])
def test_call_runs_after_prior_work_on_its_stream(op):
    import torch
    import scaled_dot_product_17_amd as sdpa
    say(f"[streams] ordering {op}")
    B, Hq, Hkv, N = 1, 8, 2, 2048
    M = 4
    q = bf16(18900, (B, Hq, M if op == "decode" else N, 128))
    k_new, v = bf16(18901, (B, Hkv, N, 128)), bf16(18902, (B, Hkv, N, 128))
    do = bf16(18903, (B, Hq, N, 128))

    def call(k):
        if op == "fwd":
            return sdpa.fwd(q, k, v, causal=True, scale=SCALE)
        if op == "decode":
            return sdpa.decode(q, k, v, causal=True, scale=SCALE)
        o, lse = sdpa.fwd(q, k, v, causal=True, scale=SCALE)
        return sdpa.bwd(q, k, v, o, lse, do, causal=True, scale=SCALE)

    expect = [to_np(t) for t in call(k_new)]
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    for _ in range(3):
        with torch.cuda.stream(s):
            k = torch.zeros_like(k_new)     # what a call run too early would see
            busy()
            k.copy_(k_new)
            got = call(k)
        s.synchronize()
        for i, (a, b) in enumerate(zip(expect, got)):
            assert np.array_equal(a, to_np(b)), f"{op}: output {i} ran out of stream order"


def test_two_threads_on_two_streams():
    import torch
    import scaled_dot_product_17_amd as sdpa
    say("[streams] two threads")
    shapes = [(2, 8, 2, 1500, True), (1, 4, 4, 3000, False)]
    ins = [(bf16(19000 + 10 * i, (B, Hq, N, 128)), bf16(19001 + 10 * i, (B, Hkv, N, 128)),
            bf16(19002 + 10 * i, (B, Hkv, N, 128)), c) for i, (B, Hq, Hkv, N, c) in enumerate(shapes)]
    expect = []
    for q, k, v, c in ins:
        expect.append([to_np(t) for t in sdpa.fwd(q, k, v, causal=c, scale=SCALE)])
    torch.cuda.synchronize()
    got, errors = {}, []

    def work(i):
        try:
            q, k, v, c = ins[i]
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                outs = [sdpa.fwd(q, k, v, causal=c, scale=SCALE) for _ in range(20)]
            s.synchronize()
            got[i] = [[to_np(t) for t in r] for r in outs]
        except Exception as e:     # reported from the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(ins))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not errors, errors
    assert all(not t.is_alive() for t in threads)
    for i in range(len(ins)):
        for r in got[i]:
            for a, b in zip(expect[i], r):
                assert np.array_equal(a, b), f"thread {i}: result differs from the sequential call"
