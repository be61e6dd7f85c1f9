"""Helpers for GPU tests: upload bf16 bit arrays, run the library, download."""
from __future__ import annotations

import numpy as np

from synth import bf16_bits_to_f32


def to_gpu(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def bf16_to_np(t) -> np.ndarray:
    """bf16 torch tensor -> float32 numpy array (exact)."""
    import torch
    return bf16_bits_to_f32(t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))


def run(q, k, v, causal, scale, lse=True):
    """Run the HIP path on bf16 bit arrays; returns (o float32 ndarray, lse ndarray|None)."""
    import torch
    import scaled_dot_product_17_amd as sdpa
    qg, kg, vg = to_gpu(q), to_gpu(k), to_gpu(v)
    o, l = sdpa.fwd(qg, kg, vg, causal=causal, scale=scale, return_lse=lse)
    torch.cuda.synchronize()
    return bf16_to_np(o), (l.cpu().numpy() if l is not None else None)


def poison_lds():
    """Leave NaN rows in the LDS of every CU: launches over NaN K and V (the
    dense forward with 8-wave and 4-wave workgroups, 512 of each, and the
    backward, whose dK/dV workgroups use most of a CU's LDS).  LDS is not
    cleared between launches, so the workgroups of the next launch inherit it."""
    import torch
    import scaled_dot_product_17_amd as sdpa
    for b, n in ((1, 8192), (8, 512)):
        q = torch.randn(b, 16, n, 128, device="cuda").to(torch.bfloat16)
        kv = torch.full((b, 16, n, 128), float("nan"), device="cuda", dtype=torch.bfloat16)
        sdpa.fwd(q, kv, kv)
    n = 4096
    q = torch.randn(1, 16, n, 128, device="cuda").to(torch.bfloat16)
    nan = torch.full((1, 16, n, 128), float("nan"), device="cuda", dtype=torch.bfloat16)
    lse = torch.zeros(1, 16, n, device="cuda")
    sdpa.bwd(q, nan, nan, nan, lse, q, n_splits=1)
    torch.cuda.synchronize()
