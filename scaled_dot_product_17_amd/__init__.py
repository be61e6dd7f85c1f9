"""MI355X (gfx950) fused scaled dot-product attention: forward (bf16 and FP8),
backward, packed variable-length forward and split-KV decode.

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
                7: "ATTN_ERR_ALIAS", 8: "ATTN_ERR_LAUNCH", 9: "ATTN_ERR_DEVICE",
                10: "ATTN_ERR_WORKSPACE", 11: "ATTN_ERR_SCRATCH"}
EXPORTED = ("attn_fwd", "attn_fwd_varlen", "attn_fwd_fp8", "attn_fwd_blocksparse", "attn_bwd", "attn_bwd_dq", "attn_bwd_dkdv",
            "attn_bwd_ws", "attn_bwd_splits", "attn_bwd_workspace_bytes", "attn_decode",
            "attn_decode_noalloc", "attn_decode_partial", "attn_decode_splits", "attn_decode_workspace_bytes", "attn_lse_merge", "attn_status_string",
            "attn_fwd_flops", "attn_bwd_flops", "attn_decode_flops")

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
            lib.attn_bwd_ws.restype = ctypes.c_int
            lib.attn_bwd_ws.argtypes = [ctypes.c_void_p] * 10 + [ctypes.c_int] * 6 + [
                ctypes.c_float, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
            lib.attn_bwd_splits.restype = ctypes.c_int
            lib.attn_bwd_splits.argtypes = [ctypes.c_int] * 7
            lib.attn_bwd_workspace_bytes.restype = ctypes.c_size_t
            lib.attn_bwd_workspace_bytes.argtypes = [ctypes.c_int] * 7
            lib.attn_fwd_varlen.restype = ctypes.c_int
            lib.attn_fwd_varlen.argtypes = [ctypes.c_void_p] * 6 + [ctypes.c_int] * 9 + [
                ctypes.c_float, ctypes.c_void_p]
            lib.attn_fwd_blocksparse.restype = ctypes.c_int
            lib.attn_fwd_blocksparse.argtypes = [ctypes.c_void_p] * 7 + [ctypes.c_int] * 8 + [
                ctypes.c_float, ctypes.c_void_p]
            lib.attn_fwd_fp8.restype = ctypes.c_int
            lib.attn_fwd_fp8.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 6 + [
                ctypes.c_float] * 4 + [ctypes.c_void_p]
            lib.attn_decode.restype = ctypes.c_int
            lib.attn_decode.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 7 + [
                ctypes.c_float, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
            lib.attn_decode_noalloc.restype = ctypes.c_int
            lib.attn_decode_noalloc.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 7 + [
                ctypes.c_float, ctypes.c_int, ctypes.c_void_p]
            lib.attn_decode_partial.restype = ctypes.c_int
            lib.attn_decode_partial.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 7 + [
                ctypes.c_float, ctypes.c_int, ctypes.c_void_p]
            lib.attn_decode_splits.restype = ctypes.c_int
            lib.attn_decode_splits.argtypes = [ctypes.c_int] * 7
            lib.attn_decode_workspace_bytes.restype = ctypes.c_size_t
            lib.attn_decode_workspace_bytes.argtypes = [ctypes.c_int] * 7
            lib.attn_lse_merge.restype = ctypes.c_int
            lib.attn_lse_merge.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                           ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_void_p]
            lib.attn_decode_flops.restype = ctypes.c_double
            lib.attn_decode_flops.argtypes = [ctypes.c_int] * 6
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


def attn_fwd_blocksparse(q, k, v, o, lse, kb_ptr, kb_idx, nnz, mask_heads, B, H_q, H_kv, N, D,
                         causal, scale, stream) -> int:
    """Direct C-ABI call with raw device pointers (ints); returns the status code."""
    return load().attn_fwd_blocksparse(q, k, v, o, lse, kb_ptr, kb_idx, int(nnz), int(mask_heads),
                                       int(B), int(H_q), int(H_kv), int(N), int(D),
                                       int(bool(causal)), float(scale), stream)


SPARSE_BLOCK = 128


def fwd_blocksparse(q, k, v, kb_ptr, kb_idx, causal: bool = False, scale: float | None = None,
                    out=None, lse=None):
    """O, LSE = attention(q, k, v) restricted to the listed 128 x 128 blocks.

    q: bf16 [B, H_q, N, D]; k, v: bf16 [B, H_kv, N, D].  kb_ptr, kb_idx: int32
    device tensors in block-compressed-row form, one list per (mask head,
    query block of 128 rows); the number of mask heads (1 or H_q) follows from
    kb_ptr's length.  Rows that see no key get O = 0 and LSE = -inf.
    """
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_bf16(name, t)
    B, Hq, N, D = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[2] != N or k.shape[3] != D:
        raise ValueError("k/v must be [B, H_kv, N, D] with q's B, N and D")
    for name, t in (("kb_ptr", kb_ptr), ("kb_idx", kb_idx)):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.int32 or t.dim() != 1 \
                or not t.is_contiguous() or t.device != q.device:
            raise ValueError(f"{name} must be a contiguous 1-D int32 tensor on q's device")
    n_blk = -(-N // SPARSE_BLOCK)
    if (kb_ptr.numel() - 1) % n_blk != 0 or kb_ptr.numel() < 2:
        raise ValueError("kb_ptr must hold mask_heads * ceil(N / 128) + 1 offsets")
    mask_heads = (kb_ptr.numel() - 1) // n_blk
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_bf16("out", out, q.shape, q.device)
    if lse is None:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        st = attn_fwd_blocksparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                  lse.data_ptr(), kb_ptr.data_ptr(),
                                  kb_idx.data_ptr() if kb_idx.numel() else None, kb_idx.numel(),
                                  mask_heads, B, Hq, k.shape[1], N, D, causal, scale, stream)
    if st != ATTN_OK:
        raise AttnError(st, status_string(st))
    return out, lse


def attn_fwd_fp8(q8, k8, v8, o, lse, B, H_q, H_kv, N, D, causal, scale, descale_q, descale_k,
                 descale_v, stream) -> int:
    """Direct C-ABI call with raw device pointers (ints); returns the status code."""
    return load().attn_fwd_fp8(q8, k8, v8, o, lse, int(B), int(H_q), int(H_kv), int(N), int(D),
                               int(bool(causal)), float(scale), float(descale_q),
                               float(descale_k), float(descale_v), stream)


def attn_fwd_varlen(q, k, v, o, lse, cu_seqlens, n_seq, max_seqlen, total, H_q, H_kv, D, causal,
                    window_left, window_right, scale, stream) -> int:
    """Direct C-ABI call with raw device pointers (ints); returns the status code."""
    return load().attn_fwd_varlen(q, k, v, o, lse, cu_seqlens, int(n_seq), int(max_seqlen),
                                  int(total), int(H_q), int(H_kv), int(D), int(bool(causal)),
                                  int(window_left), int(window_right), float(scale), stream)


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


def attn_bwd_ws(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H_q, H_kv, N, D, causal, scale,
                n_splits, workspace, workspace_bytes, stream) -> int:
    return load().attn_bwd_ws(q, k, v, o, dout, lse, dq, dk, dv, delta, int(B), int(H_q), int(H_kv),
                              int(N), int(D), int(bool(causal)), float(scale), int(n_splits),
                              workspace, int(workspace_bytes), stream)


def attn_bwd_splits(B, H_q, H_kv, N, D, causal=False, n_splits=0) -> int:
    return load().attn_bwd_splits(int(B), int(H_q), int(H_kv), int(N), int(D), int(bool(causal)),
                                  int(n_splits))


def attn_bwd_workspace_bytes(B, H_q, H_kv, N, D, causal=False, n_splits=0) -> int:
    return load().attn_bwd_workspace_bytes(int(B), int(H_q), int(H_kv), int(N), int(D),
                                           int(bool(causal)), int(n_splits))


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


def fwd_fp8(q8, k8, v8, descale_q: float = 1.0, descale_k: float = 1.0, descale_v: float = 1.0,
            causal: bool = False, scale: float | None = None, out=None, lse=None,
            return_lse: bool = True):
    """O, LSE = attention(descale_q*q8, descale_k*k8, descale_v*v8) on the current
    torch stream, with q8, k8, v8 e4m3 codes (torch.uint8 or torch.float8_e4m3fn,
    [B, H_q, N, D] and [B, H_kv, N, D], contiguous, on one GPU).  O is bf16
    [B, H_q, N, D], lse fp32 [B, H_q, N].  ``scale`` defaults to 1/sqrt(D)."""
    import torch

    for name, t in (("q8", q8), ("k8", k8), ("v8", v8)):
        if not isinstance(t, torch.Tensor) or t.dim() != 4 or \
                t.dtype not in (torch.uint8, torch.float8_e4m3fn):
            raise ValueError(f"{name} must be a 4-D torch.uint8 or torch.float8_e4m3fn tensor")
        if not t.is_cuda:
            raise ValueError(f"{name} must be on a GPU")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if k8.shape != v8.shape:
        raise ValueError("k8 and v8 must have the same shape")
    B, Hq, N, D = q8.shape
    if k8.shape[0] != B or k8.shape[2] != N or k8.shape[3] != D:
        raise ValueError("k8/v8 must be [B, H_kv, N, D] with q8's B, N and D")
    if not (q8.device == k8.device == v8.device):
        raise ValueError("q8, k8 and v8 must be on the same device")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, Hq, N, D), dtype=torch.bfloat16, device=q8.device)
    else:
        _check_bf16("out", out, (B, Hq, N, D), q8.device)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q8.device)
    elif lse is not None and (lse.shape != (B, Hq, N) or lse.dtype != torch.float32
                              or not lse.is_contiguous() or lse.device != q8.device):
        raise ValueError("lse must be a contiguous fp32 [B, H_q, N] tensor on q8's device")
    with torch.cuda.device(q8.device):
        stream = torch.cuda.current_stream(q8.device).cuda_stream
        st = attn_fwd_fp8(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), out.data_ptr(),
                          lse.data_ptr() if lse is not None else None, B, Hq, k8.shape[1], N, D,
                          causal, scale, descale_q, descale_k, descale_v, stream)
    if st != ATTN_OK:
        raise AttnError(st, status_string(st))
    return out, lse


def bwd(q, k, v, o, lse, dout, causal: bool = False, scale: float | None = None,
        dq=None, dk=None, dv=None, delta=None, n_splits: int = 0, workspace=None):
    """dQ, dK, dV of attention on the current torch stream of q's device.

    q, o, dout: bf16 [B, H_q, N, D]; k, v: bf16 [B, H_kv, N, D]; lse: fp32
    [B, H_q, N] from ``fwd`` with the same causal and scale.  Output buffers may
    be given to avoid allocation.  Returns (dq, dk, dv, delta) with delta the
    fp32 [B, H_q, N] row sums dO . O.  When the library splits the dK/dV step
    over a group's query heads (attn_bwd_splits; n_splits <= 0: its choice)
    this calls attn_bwd_ws with `workspace` (a uint8 tensor on q's device, or
    allocated here), else attn_bwd.
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
    ns = attn_bwd_splits(B, Hq, Hkv, N, D, causal, n_splits)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(),
                B, Hq, Hkv, N, D, causal, scale)
        if ns > 1:
            need = attn_bwd_workspace_bytes(B, Hq, Hkv, N, D, causal, ns)
            if workspace is None:
                workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
            elif not isinstance(workspace, torch.Tensor) or workspace.device != q.device or \
                    not workspace.is_contiguous():
                raise ValueError("workspace must be a contiguous tensor on q's device")
            st = attn_bwd_ws(*args, ns, workspace.data_ptr(),
                             workspace.numel() * workspace.element_size(), stream)
        else:
            st = attn_bwd(*args, stream)
    if st != ATTN_OK:
        raise AttnError(st, status_string(st))
    return dq, dk, dv, delta


def attn_decode(q, k, v, o, lse, B, H_q, H_kv, M, L, D, causal, scale, n_splits, workspace,
                workspace_bytes, stream) -> int:
    """Direct C-ABI call with raw device pointers (ints); returns the status code."""
    return load().attn_decode(q, k, v, o, lse, int(B), int(H_q), int(H_kv), int(M), int(L),
                              int(D), int(bool(causal)), float(scale), int(n_splits), workspace,
                              int(workspace_bytes), stream)


def attn_decode_noalloc(q, k, v, o, lse, B, H_q, H_kv, M, L, D, causal, scale, n_splits,
                        stream) -> int:
    """Direct C-ABI call (decode with the library's fixed scratch array, no
    workspace); returns the status code."""
    return load().attn_decode_noalloc(q, k, v, o, lse, int(B), int(H_q), int(H_kv), int(M),
                                      int(L), int(D), int(bool(causal)), float(scale),
                                      int(n_splits), stream)


# bytes of the fixed scratch array attn_decode_noalloc uses (ATTN_DECODE_SCRATCH_BYTES)
DECODE_SCRATCH_BYTES = 16 << 20


def attn_decode_partial(q, k, v, o_part, lse_part, B, H_q, H_kv, M, L, D, causal, scale,
                        n_splits, stream) -> int:
    """Direct C-ABI call (the split kernel alone); returns the status code."""
    return load().attn_decode_partial(q, k, v, o_part, lse_part, int(B), int(H_q), int(H_kv),
                                      int(M), int(L), int(D), int(bool(causal)), float(scale),
                                      int(n_splits), stream)


def attn_decode_splits(B, H_q, H_kv, M, L, D, n_splits=0) -> int:
    return int(load().attn_decode_splits(int(B), int(H_q), int(H_kv), int(M), int(L), int(D),
                                         int(n_splits)))


def attn_decode_workspace_bytes(B, H_q, H_kv, M, L, D, n_splits=0) -> int:
    return int(load().attn_decode_workspace_bytes(int(B), int(H_q), int(H_kv), int(M), int(L),
                                                  int(D), int(n_splits)))


def attn_lse_merge(o_part, lse_part, rows, n_parts, D, o, lse, stream) -> int:
    """Direct C-ABI call with raw device pointers (ints); returns the status code."""
    return load().attn_lse_merge(o_part, lse_part, int(rows), int(n_parts), int(D), o, lse,
                                 stream)


def attn_decode_flops(B, H_q, M, L, D, causal) -> float:
    return load().attn_decode_flops(int(B), int(H_q), int(M), int(L), int(D), int(bool(causal)))


def decode(q, k, v, causal: bool = False, scale: float | None = None, n_splits: int = 0,
           out=None, lse=None, workspace=None):
    """O, LSE of M query rows against an L-key cache, on q's current stream.

    q: bf16 [B, H_q, M, D]; k, v: bf16 [B, H_kv, L, D].  With ``causal`` row i
    sees keys 0..L-M+i.  ``workspace``: optional uint8 device tensor of at least
    attn_decode_workspace_bytes(...) bytes.  Returns (o, lse).
    """
    import torch

    _check_bf16("q", q)
    B, Hq, M, D = q.shape
    _check_bf16("k", k, device=q.device)
    Hkv, L = k.shape[1], k.shape[2]
    if k.shape[0] != B or k.shape[3] != D:
        raise ValueError("k/v must be [B, H_kv, L, D] with q's B and D")
    _check_bf16("v", v, k.shape, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = torch.empty_like(q) if out is None else out
    _check_bf16("out", out, q.shape, q.device)
    if lse is None:
        lse = torch.empty((B, Hq, M), dtype=torch.float32, device=q.device)
    elif lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, M) or \
            not lse.is_contiguous() or lse.device != q.device:
        raise ValueError("lse must be a contiguous fp32 [B, H_q, M] tensor on q's device")
    need = attn_decode_workspace_bytes(B, Hq, Hkv, M, L, D, n_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        st = attn_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                         lse.data_ptr(), B, Hq, Hkv, M, L, D, causal, scale, n_splits,
                         workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                         stream)
    if st != ATTN_OK:
        raise AttnError(st, status_string(st))
    return out, lse


def lse_merge(o_part, lse_part, out=None, lse=None):
    """Merge fp32 partials o_part [rows, P, D], lse_part [rows, P] into bf16
    O [rows, D] and fp32 LSE [rows] on the current stream."""
    import torch

    if o_part.dtype != torch.float32 or o_part.dim() != 3 or not o_part.is_contiguous() \
            or not o_part.is_cuda:
        raise ValueError("o_part must be a contiguous fp32 [rows, P, D] GPU tensor")
    rows, P, D = o_part.shape
    if lse_part.dtype != torch.float32 or tuple(lse_part.shape) != (rows, P) or \
            not lse_part.is_contiguous() or lse_part.device != o_part.device:
        raise ValueError("lse_part must be a contiguous fp32 [rows, P] tensor on o_part's device")
    out = torch.empty((rows, D), dtype=torch.bfloat16, device=o_part.device) if out is None else out
    lse = torch.empty((rows,), dtype=torch.float32, device=o_part.device) if lse is None else lse
    with torch.cuda.device(o_part.device):
        stream = torch.cuda.current_stream(o_part.device).cuda_stream
        st = attn_lse_merge(o_part.data_ptr(), lse_part.data_ptr(), rows, P, D, out.data_ptr(),
                            lse.data_ptr(), stream)
    if st != ATTN_OK:
        raise AttnError(st, status_string(st))
    return out, lse


def fwd_varlen(q, k, v, cu_seqlens, max_seqlen: int, causal: bool = False,
               scale: float | None = None, window=(-1, -1), out=None, lse=None):
    """O, LSE of a packed batch: q bf16 [H_q, total, D], k, v bf16 [H_kv, total, D],
    cu_seqlens int32 [n_seq + 1] on the same GPU.  ``window`` = (left, right):
    row i sees keys i-left .. i+right of its sequence (negative: unbounded).
    Returns (o, lse) with lse fp32 [H_q, total]."""
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or t.dim() != 3 \
                or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 3-D bf16 GPU tensor")
    Hq, total, D = q.shape
    if k.shape != v.shape or k.shape[1:] != q.shape[1:] or k.device != q.device or \
            v.device != q.device:
        raise ValueError("k, v must be [H_kv, total, D] like q, on q's device")
    if not isinstance(cu_seqlens, torch.Tensor) or cu_seqlens.dtype != torch.int32 or \
            cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2 or cu_seqlens.device != q.device \
            or not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous int32 [n_seq + 1] tensor on q's device")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = torch.empty_like(q) if out is None else out
    if lse is None:
        lse = torch.empty((Hq, total), dtype=torch.float32, device=q.device)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        st = attn_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                             lse.data_ptr(), cu_seqlens.data_ptr(), cu_seqlens.numel() - 1,
                             max_seqlen, total, Hq, k.shape[0], D, causal, window[0], window[1],
                             scale, stream)
    if st != ATTN_OK:
        raise AttnError(st, status_string(st))
    return out, lse
