"""Stale LDS is never read.

The kernels clear their LDS rings only when a size is ragged (a tail block
with rows past the end). Otherwise every ring slot a kernel reads was filled
by its own copies first. These tests fill the LDS of every CU with NaN rows,
by launching kernels over NaN inputs. They then check that launches with
whole-block sizes (FP8 forward, backward with and without the K/V-head split,
split-KV decode) reproduce their earlier results bitwise and stay finite.
Each launch's parity against the oracle is covered by that path's own tests.
"""
import math
import sys

import numpy as np
import pytest

import synth
from tests.gpu_util import bf16_to_np, poison_lds, to_gpu

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


def same_after_poison(run, what):
    first = run()
    poison_lds()
    after = run()
    for i, (a, b) in enumerate(zip(first, after)):
        assert np.array_equal(a, b, equal_nan=True), f"{what}: output {i} changed after stale LDS"
        assert np.all(np.isfinite(b) | np.isneginf(b)), f"{what}: output {i} not finite"


def to_np(t):
    import torch
    return bf16_to_np(t) if t.dtype == torch.bfloat16 else t.cpu().numpy()


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_whole_blocks(causal):
    import torch
    import scaled_dot_product_17_amd as sdpa
    B, Hq, Hkv, N = 2, 8, 2, 1024          # N a multiple of the 64-key block
    say(f"[stale lds] fp8 causal={causal}")
    d = synth.FP8_DESCALE
    q8, k8, v8 = (torch.from_numpy(synth.normal_e4m3(18000 + i, (B, h, N, 128), d)).cuda()
                  for i, h in enumerate((Hq, Hkv, Hkv)))

    def run():
        o, lse = sdpa.fwd_fp8(q8, k8, v8, d, d, d, causal=causal, scale=SCALE)
        torch.cuda.synchronize()
        return [to_np(o), to_np(lse)]

    same_after_poison(run, f"fp8 causal={causal}")


@pytest.mark.parametrize("n_splits", [1, 0])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_whole_blocks(causal, n_splits):
    import torch
    import scaled_dot_product_17_amd as sdpa
    B, Hq, Hkv, N = 1, 8, 1, 1024          # MQA: the automatic split count is above 1
    say(f"[stale lds] bwd causal={causal} n_splits={n_splits}")
    q, k, v, do = (to_gpu(synth.normal_bf16(18100 + i, (B, h, N, 128)))
                   for i, h in enumerate((Hq, Hkv, Hkv, Hq)))
    o, lse = sdpa.fwd(q, k, v, causal=causal, scale=SCALE)

    def run():
        outs = sdpa.bwd(q, k, v, o, lse, do, causal=causal, scale=SCALE, n_splits=n_splits)
        torch.cuda.synchronize()
        return [to_np(t) for t in outs]

    same_after_poison(run, f"bwd causal={causal} n_splits={n_splits}")


@pytest.mark.parametrize("M,causal", [(1, False), (4, True)])
def test_decode_whole_blocks(M, causal):
    import torch
    import scaled_dot_product_17_amd as sdpa
    B, Hq, Hkv, L = 2, 16, 2, 2048          # L a multiple of the 32-key block
    say(f"[stale lds] decode M={M} causal={causal}")
    q = to_gpu(synth.normal_bf16(18200, (B, Hq, M, 128)))
    k = to_gpu(synth.normal_bf16(18201, (B, Hkv, L, 128)))
    v = to_gpu(synth.normal_bf16(18202, (B, Hkv, L, 128)))

    def run():
        o, lse = sdpa.decode(q, k, v, causal=causal, scale=SCALE)
        torch.cuda.synchronize()
        return [to_np(o), to_np(lse)]

    same_after_poison(run, f"decode M={M} causal={causal}")
