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
