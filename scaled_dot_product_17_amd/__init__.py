"""MI355X (gfx950) fused scaled dot-product attention, forward and backward.

Thin Python binding over the C ABI declared in ``include/attn.h``: argument
marshalling only.  Every step of the computation runs in the HIP kernels of
``libattn.so``; torch provides device memory and streams.  There is no CPU
or fallback path: if the library is missing or the GPU is not a gfx950 the
calls raise.
"""
from __future__ import annotations

import ctypes
import math
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libattn.so")

ATTN_OK = 0
STATUS_NAMES = {0: "ATTN_OK", 1: "ATTN_ERR_NULL", 2: "ATTN_ERR_SHAPE", 3: "ATTN_ERR_GQA",
                4: "ATTN_ERR_HEAD_DIM", 5: "ATTN_ERR_SCALE", 6: "ATTN_ERR_ALIGN",
                7: "ATTN_ERR_ALIAS", 8: "ATTN_ERR_LAUNCH", 9: "ATTN_ERR_DEVICE"}
EXPORTED = ("attn_fwd", "attn_bwd", "attn_bwd_dq", "attn_bwd_dkdv", "attn_status_string",
            "attn_fwd_flops", "attn_bwd_flops")

_lock = threading.Lock()
_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the built HIP library (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(path):
                raise ImportError(f"{path} is missing: build it first "
                                  "(python -m scaled_dot_product_17_amd._build)")
            lib = ctypes.CDLL(path)
            lib.attn_fwd.restype = ctypes.c_int
            lib.attn_fwd.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 6 + [
                ctypes.c_float, ctypes.c_void_p]
            lib.attn_status_string.restype = ctypes.c_char_p
            lib.attn_status_string.argtypes = [ctypes.c_int]
            lib.attn_fwd_flops.restype = ctypes.c_double
            lib.attn_fwd_flops.argtypes = [ctypes.c_int] * 5
            lib.attn_bwd.restype = ctypes.c_int
            lib.attn_bwd.argtypes = [ctypes.c_void_p] * 10 + [ctypes.c_int] * 6 + [
                ctypes.c_float, ctypes.c_void_p]
            lib.attn_bwd_dq.restype = ctypes.c_int
            lib.attn_bwd_dq.argtypes = [ctypes.c_void_p] * 8 + [ctypes.c_int] * 6 + [
                ctypes.c_float, ctypes.c_void_p]
            lib.attn_bwd_dkdv.restype = ctypes.c_int
            lib.attn_bwd_dkdv.argtypes = [ctypes.c_void_p] * 8 + [ctypes.c_int] * 6 + [
                ctypes.c_float, ctypes.c_void_p]
            lib.attn_bwd_flops.restype = ctypes.c_double
            lib.attn_bwd_flops.argtypes = [ctypes.c_int] * 5
            _lib = lib
    return _lib


def status_string(status: int) -> str:
    return load().attn_status_string(int(status)).decode()


def attn_fwd(q, k, v, o, lse, B, H_q, H_kv, N, D, causal, scale, stream) -> int:
    """Direct C-ABI call with raw device pointers (ints); returns the status code."""
    return load().attn_fwd(q, k, v, o, lse, int(B), int(H_q), int(H_kv), int(N), int(D),
                           int(bool(causal)), float(scale), stream)


def attn_fwd_flops(B, H_q, N, D, causal) -> float:
    return load().attn_fwd_flops(int(B), int(H_q), int(N), int(D), int(bool(causal)))


def attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H_q, H_kv, N, D, causal, scale,
             stream) -> int:
    """Direct C-ABI call with raw device pointers (ints); returns the status code."""
    return load().attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, int(B), int(H_q),
                           int(H_kv), int(N), int(D), int(bool(causal)), float(scale), stream)


def attn_bwd_dq(q, k, v, o, dout, lse, dq, delta, B, H_q, H_kv, N, D, causal, scale,
                stream) -> int:
    """Direct C-ABI call (the dQ kernel alone); returns the status code."""
    return load().attn_bwd_dq(q, k, v, o, dout, lse, dq, delta, int(B), int(H_q), int(H_kv),
                              int(N), int(D), int(bool(causal)), float(scale), stream)


def attn_bwd_dkdv(q, k, v, dout, lse, delta, dk, dv, B, H_q, H_kv, N, D, causal, scale,
                  stream) -> int:
    """Direct C-ABI call (the dK/dV kernel alone); returns the status code."""
    return load().attn_bwd_dkdv(q, k, v, dout, lse, delta, dk, dv, int(B), int(H_q),
                                int(H_kv), int(N), int(D), int(bool(causal)), float(scale),
                                stream)


def attn_bwd_flops(B, H_q, N, D, causal) -> float:
    return load().attn_bwd_flops(int(B), int(H_q), int(N), int(D), int(bool(causal)))


def _check_bf16(name, t, shape=None, device=None):
    import torch

    if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or t.dim() != 4:
        raise ValueError(f"{name} must be a 4-D torch.bfloat16 tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}")


def fwd(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None,
        return_lse: bool = True):
    """O, LSE = attention(q, k, v) on the current torch stream of q's device.

    q: bf16 [B, H_q, N, D]; k, v: bf16 [B, H_kv, N, D]; contiguous, on one GPU.
    ``scale`` defaults to 1/sqrt(D).  ``out``/``lse`` may be given to avoid
    allocation.  Returns (o, lse) with lse fp32 [B, H_q, N] (None when
    return_lse is False and no lse buffer was given).
    """
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or t.dim() != 4:
            raise ValueError(f"{name} must be a 4-D torch.bfloat16 tensor")
        if not t.is_cuda:
            raise ValueError(f"{name} must be on a GPU")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if k.shape != v.shape:
        raise ValueError("k and v must have the same shape")
    B, Hq, N, D = q.shape
    if k.shape[0] != B or k.shape[2] != N or k.shape[3] != D:
        raise ValueError("k/v must be [B, H_kv, N, D] with q's B, N and D")
    Hkv = k.shape[1]
    if not (q.device == k.device == v.device):
        raise ValueError("q, k and v must be on the same device")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != torch.bfloat16 or not out.is_contiguous() \
            or out.device != q.device:
        raise ValueError("out must be a contiguous bf16 tensor shaped like q on q's device")
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    elif lse is not None and (lse.shape != (B, Hq, N) or lse.dtype != torch.float32
                              or not lse.is_contiguous() or lse.device != q.device):
        raise ValueError("lse must be a contiguous fp32 [B, H_q, N] tensor on q's device")
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        st = attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                      lse.data_ptr() if lse is not None else None, B, Hq, Hkv, N, D,
                      causal, scale, stream)
    if st != ATTN_OK:
        raise AttnError(st, status_string(st))
    return out, lse


def bwd(q, k, v, o, lse, dout, causal: bool = False, scale: float | None = None,
        dq=None, dk=None, dv=None, delta=None):
    """dQ, dK, dV of attention on the current torch stream of q's device.

    q, o, dout: bf16 [B, H_q, N, D]; k, v: bf16 [B, H_kv, N, D]; lse: fp32
    [B, H_q, N] from ``fwd`` with the same causal and scale.  Output buffers may
    be given to avoid allocation.  Returns (dq, dk, dv, delta) with delta the
    fp32 [B, H_q, N] row sums dO . O.
    """
    import torch

    _check_bf16("q", q)
    B, Hq, N, D = q.shape
    _check_bf16("k", k, device=q.device)
    Hkv = k.shape[1]
    if k.shape[0] != B or k.shape[2] != N or k.shape[3] != D:
        raise ValueError("k/v must be [B, H_kv, N, D] with q's B, N and D")
    _check_bf16("v", v, k.shape, q.device)
    _check_bf16("o", o, q.shape, q.device)
    _check_bf16("dout", dout, q.shape, q.device)
    if not isinstance(lse, torch.Tensor) or lse.dtype != torch.float32 or \
            tuple(lse.shape) != (B, Hq, N) or not lse.is_contiguous() or lse.device != q.device:
        raise ValueError("lse must be a contiguous fp32 [B, H_q, N] tensor on q's device")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _check_bf16("dq", dq, q.shape, q.device)
    _check_bf16("dk", dk, k.shape, q.device)
    _check_bf16("dv", dv, k.shape, q.device)
    if delta is None:
        delta = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    elif delta.dtype != torch.float32 or tuple(delta.shape) != (B, Hq, N) or \
            not delta.is_contiguous() or delta.device != q.device:
        raise ValueError("delta must be a contiguous fp32 [B, H_q, N] tensor on q's device")
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        st = attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                      lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                      delta.data_ptr(), B, Hq, Hkv, N, D, causal, scale, stream)
    if st != ATTN_OK:
        raise AttnError(st, status_string(st))
    return dq, dk, dv, delta
