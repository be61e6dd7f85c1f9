"""fp64 CPU oracle for the attention forward pass.

TEST INFRASTRUCTURE ONLY: used by ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py``.  The product library never imports,
links or calls anything here, and nothing here imports the product package.

``attn_ref`` wraps the C routine in ``attn_ref.c`` (the plain definition,
softmax(scale * Q K^T [causal]) V and its log-sum-exp, in double precision).
``attn_bwd_ref`` wraps ``attn_bwd_ref.c`` (the chain rule through that
definition: dQ, dK, dV for a given dO, in double precision).
``attn_varlen_ref`` wraps ``attn_varlen_ref.c`` (a packed batch of variable-length
sequences with an optional sliding window).
``attn_decode_ref`` and ``attn_lse_merge_ref`` wrap ``attn_decode_ref.c`` (M
query rows against an L-key cache, and the exact merge of partial results by
their log-sum-exp).
``attn_fp8_ref`` wraps ``attn_fp8_ref.c`` (the forward on e4m3 inputs with
per-tensor scales, evaluated exactly on the values the codes stand for) and
``e4m3_decode`` its code-to-value rule.
``attn_blocksparse_ref`` wraps ``attn_blocksparse_ref.c`` (the forward with a
block-sparse mask given as per-query-block lists of key blocks).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRCS = [os.path.join(_HERE, n) for n in
         ("attn_ref.c", "attn_bwd_ref.c", "attn_decode_ref.c", "attn_varlen_ref.c",
          "attn_fp8_ref.c", "attn_blocksparse_ref.c")]
_LIB = os.path.join(_HERE, "libattn_ref.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with the host C compiler (no fast-math: IEEE double)."""
    if force or not os.path.exists(_LIB) or \
            os.path.getmtime(_LIB) < max(os.path.getmtime(s) for s in _SRCS):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-fno-fast-math",
               "-ffp-contract=off", "-o", tmp] + _SRCS + ["-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _bind(path: str):
    lib = ctypes.CDLL(path)
    fn = lib.attn_ref_f64
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 6 + [
        ctypes.c_double, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64]
    if hasattr(lib, "attn_bwd_ref_f64"):
        bw = lib.attn_bwd_ref_f64
        bw.restype = ctypes.c_int
        bw.argtypes = [ctypes.c_void_p] * 10 + [ctypes.c_int] * 6 + [
            ctypes.c_double, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64]
        bk = lib.attn_bwd_ref_keys_f64
        bk.restype = ctypes.c_int
        bk.argtypes = [ctypes.c_void_p] * 8 + [ctypes.c_int] * 6 + [
            ctypes.c_double, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64]
    if hasattr(lib, "attn_varlen_ref_f64"):
        vl = lib.attn_varlen_ref_f64
        vl.restype = ctypes.c_int
        vl.argtypes = [ctypes.c_void_p] * 6 + [ctypes.c_int] * 7 + [ctypes.c_double]
    if hasattr(lib, "attn_fp8_ref_f64"):
        f8 = lib.attn_fp8_ref_f64
        f8.restype = ctypes.c_int
        f8.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_double] * 3 + [ctypes.c_void_p] * 4 + [
            ctypes.c_int] * 6 + [ctypes.c_double] * 3 + [ctypes.c_void_p, ctypes.c_int64]
        dec = lib.e4m3_decode
        dec.restype = ctypes.c_double
        dec.argtypes = [ctypes.c_uint8]
    if hasattr(lib, "attn_blocksparse_ref_f64"):
        bs = lib.attn_blocksparse_ref_f64
        bs.restype = ctypes.c_int
        bs.argtypes = [ctypes.c_void_p] * 7 + [ctypes.c_int] * 8 + [ctypes.c_double, ctypes.c_void_p,
                                                                     ctypes.c_int64]
    if hasattr(lib, "attn_decode_ref_f64"):
        dc = lib.attn_decode_ref_f64
        dc.restype = ctypes.c_int
        dc.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 7 + [ctypes.c_double]
        mg = lib.attn_lse_merge_ref_f64
        mg.restype = ctypes.c_int
        mg.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                       ctypes.c_void_p, ctypes.c_void_p]
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB):
                build(force=False)
            _lib = _bind(_LIB)
    return _lib


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def attn_ref(q, k, v, causal: bool, scale: float, rows=None, n_threads: int | None = None):
    """Oracle forward pass.

    q: uint16 bf16 bits [B, H_q, N, D]; k, v: uint16 bf16 bits [B, H_kv, N, D].
    ``scale`` is used exactly as the double given (pass float(np.float32(s)) to
    mirror an fp32 scale).  ``rows``: optional int64 flat row ids
    ((b*H_q + h)*N + i); then the result holds just those rows.

    Returns (o, lse) as float64: o [B, H_q, N, D] and lse [B, H_q, N], or
    o [len(rows), D] and lse [len(rows)].
    """
    return call_lib(_load(), q, k, v, causal, scale, rows, n_threads)


def call_lib(lib, q, k, v, causal, scale, rows=None, n_threads=None):
    """``attn_ref`` against an explicitly loaded oracle library (see ``_bind``)."""
    q = np.ascontiguousarray(q, dtype=np.uint16)
    k = np.ascontiguousarray(k, dtype=np.uint16)
    v = np.ascontiguousarray(v, dtype=np.uint16)
    if q.ndim != 4 or k.ndim != 4 or v.shape != k.shape:
        raise ValueError("q must be [B,H_q,N,D], k and v [B,H_kv,N,D]")
    B, Hq, N, D = q.shape
    Hkv = k.shape[1]
    if k.shape[0] != B or k.shape[2] != N or k.shape[3] != D:
        raise ValueError("shape mismatch between q and k/v")
    if rows is None:
        o = np.empty((B, Hq, N, D), dtype=np.float64)
        lse = np.empty((B, Hq, N), dtype=np.float64)
        rows_p, n_rows = None, 0
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1)
        o = np.empty((rows.size, D), dtype=np.float64)
        lse = np.empty((rows.size,), dtype=np.float64)
        rows_p, n_rows = rows.ctypes.data, rows.size
    nt = default_threads() if n_threads is None else int(n_threads)
    rc = lib.attn_ref_f64(q.ctypes.data, k.ctypes.data, v.ctypes.data, o.ctypes.data,
                          lse.ctypes.data, B, Hq, Hkv, N, D, int(bool(causal)),
                          float(scale), nt, rows_p, n_rows)
    if rc != 0:
        raise ValueError(f"attn_ref_f64 failed with code {rc}")
    return o, lse


def attn_bwd_ref(q, k, v, do, causal: bool, scale: float, rows=None, mags: bool = False,
                 n_threads: int | None = None, keys=None):
    """Oracle backward pass (gradients of the forward for an output gradient dO).

    q, do: uint16 bf16 bits [B, H_q, N, D]; k, v: uint16 bf16 bits [B, H_kv, N, D].
    Returns (dq, dk, dv) as float64 ([B,H_q,N,D], [B,H_kv,N,D], [B,H_kv,N,D]).
    ``rows``: optional int64 flat row ids; then only dq is computed and returned,
    as [len(rows), D].  ``keys``: optional int64 flat key ids ((b*H_kv + kv)*N + j);
    then only (dk, dv) of those keys are returned, as [len(keys), D] each.
    ``mags``: also return the error-scale sums (same shapes, appended after the
    gradients) that the parity tolerance is built from.
    """
    return call_bwd_lib(_load(), q, k, v, do, causal, scale, rows, mags, n_threads, keys)


def call_bwd_lib(lib, q, k, v, do, causal, scale, rows=None, mags=False, n_threads=None,
                 keys=None):
    """``attn_bwd_ref`` against an explicitly loaded oracle library (see ``_bind``)."""
    q = np.ascontiguousarray(q, dtype=np.uint16)
    k = np.ascontiguousarray(k, dtype=np.uint16)
    v = np.ascontiguousarray(v, dtype=np.uint16)
    do = np.ascontiguousarray(do, dtype=np.uint16)
    if q.ndim != 4 or k.ndim != 4 or v.shape != k.shape or do.shape != q.shape:
        raise ValueError("q, do must be [B,H_q,N,D], k and v [B,H_kv,N,D]")
    B, Hq, N, D = q.shape
    Hkv = k.shape[1]
    if k.shape[0] != B or k.shape[2] != N or k.shape[3] != D:
        raise ValueError("shape mismatch between q and k/v")
    nt = default_threads() if n_threads is None else int(n_threads)
    if keys is not None:
        if rows is not None:
            raise ValueError("give rows or keys, not both")
        keys = np.ascontiguousarray(keys, dtype=np.int64).reshape(-1)
        dk = np.empty((keys.size, D))
        dv = np.empty((keys.size, D))
        mdk = np.empty_like(dk) if mags else None
        mdv = np.empty_like(dv) if mags else None
        rc = lib.attn_bwd_ref_keys_f64(q.ctypes.data, k.ctypes.data, v.ctypes.data, do.ctypes.data,
                                       dk.ctypes.data, dv.ctypes.data,
                                       None if mdk is None else mdk.ctypes.data,
                                       None if mdv is None else mdv.ctypes.data,
                                       B, Hq, Hkv, N, D, int(bool(causal)), float(scale), nt,
                                       keys.ctypes.data, keys.size)
        if rc != 0:
            raise ValueError(f"attn_bwd_ref_keys_f64 failed with code {rc}")
        return (dk, dv, mdk, mdv) if mags else (dk, dv)
    if rows is None:
        dq = np.empty((B, Hq, N, D))
        dk = np.empty((B, Hkv, N, D))
        dv = np.empty((B, Hkv, N, D))
        out = [dq, dk, dv]
        mg = [np.empty_like(a) for a in out] if mags else [None] * 3
        rows_p, n_rows = None, 0
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1)
        dq = np.empty((rows.size, D))
        out = [dq]
        mg = [np.empty_like(dq) if mags else None, None, None]
        rows_p, n_rows = rows.ctypes.data, rows.size
    ptr = lambda a: None if a is None else a.ctypes.data
    rc = lib.attn_bwd_ref_f64(q.ctypes.data, k.ctypes.data, v.ctypes.data, do.ctypes.data,
                              ptr(out[0]), ptr(out[1]) if rows is None else None,
                              ptr(out[2]) if rows is None else None,
                              ptr(mg[0]), ptr(mg[1]), ptr(mg[2]),
                              B, Hq, Hkv, N, D, int(bool(causal)), float(scale), nt,
                              rows_p, n_rows)
    if rc != 0:
        raise ValueError(f"attn_bwd_ref_f64 failed with code {rc}")
    if rows is not None:
        return (dq, mg[0]) if mags else dq
    return tuple(out + mg) if mags else tuple(out)


def attn_decode_ref(q, k, v, causal: bool, scale: float):
    """Oracle decode: q bf16 bits [B, H_q, M, D] against k, v bf16 bits
    [B, H_kv, L, D]; with ``causal`` row i sees keys 0..L-M+i.  Returns (o, lse)
    as float64 [B, H_q, M, D] and [B, H_q, M]."""
    return call_decode_lib(_load(), q, k, v, causal, scale)


def call_decode_lib(lib, q, k, v, causal, scale):
    q = np.ascontiguousarray(q, dtype=np.uint16)
    k = np.ascontiguousarray(k, dtype=np.uint16)
    v = np.ascontiguousarray(v, dtype=np.uint16)
    if q.ndim != 4 or k.ndim != 4 or v.shape != k.shape:
        raise ValueError("q must be [B,H_q,M,D], k and v [B,H_kv,L,D]")
    B, Hq, M, D = q.shape
    Hkv, L = k.shape[1], k.shape[2]
    if k.shape[0] != B or k.shape[3] != D:
        raise ValueError("shape mismatch between q and k/v")
    o = np.empty((B, Hq, M, D))
    lse = np.empty((B, Hq, M))
    rc = lib.attn_decode_ref_f64(q.ctypes.data, k.ctypes.data, v.ctypes.data, o.ctypes.data,
                                 lse.ctypes.data, B, Hq, Hkv, M, L, D, int(bool(causal)),
                                 float(scale))
    if rc != 0:
        raise ValueError(f"attn_decode_ref_f64 failed with code {rc}")
    return o, lse


def attn_lse_merge_ref(o_part, lse_part):
    """Oracle merge: o_part [rows, P, D] and lse_part [rows, P] (float64; -inf
    marks an empty part) -> (o [rows, D], lse [rows])."""
    return call_merge_lib(_load(), o_part, lse_part)


def call_merge_lib(lib, o_part, lse_part):
    o_part = np.ascontiguousarray(o_part, dtype=np.float64)
    lse_part = np.ascontiguousarray(lse_part, dtype=np.float64)
    if o_part.ndim != 3 or lse_part.shape != o_part.shape[:2]:
        raise ValueError("o_part must be [rows, P, D] and lse_part [rows, P]")
    rows, P, D = o_part.shape
    o = np.empty((rows, D))
    lse = np.empty((rows,))
    rc = lib.attn_lse_merge_ref_f64(o_part.ctypes.data, lse_part.ctypes.data, rows, P, D,
                                    o.ctypes.data, lse.ctypes.data)
    if rc != 0:
        raise ValueError(f"attn_lse_merge_ref_f64 failed with code {rc}")
    return o, lse


def attn_varlen_ref(q, k, v, cu_seqlens, causal: bool, scale: float, left: int = -1,
                    right: int = -1):
    """Oracle forward over a packed batch: q bf16 bits [H_q, total, D], k, v
    [H_kv, total, D], cu_seqlens int32 [n_seq + 1]; row i sees keys j of its own
    sequence with i-left <= j <= i+right (negative: unbounded) and, with
    ``causal``, j <= i.  Returns (o, lse) as float64 [H_q, total, D], [H_q, total]."""
    return call_varlen_lib(_load(), q, k, v, cu_seqlens, causal, scale, left, right)


def call_varlen_lib(lib, q, k, v, cu_seqlens, causal, scale, left=-1, right=-1):
    q = np.ascontiguousarray(q, dtype=np.uint16)
    k = np.ascontiguousarray(k, dtype=np.uint16)
    v = np.ascontiguousarray(v, dtype=np.uint16)
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    if q.ndim != 3 or k.ndim != 3 or v.shape != k.shape or k.shape[1:] != q.shape[1:]:
        raise ValueError("q must be [H_q, total, D], k and v [H_kv, total, D]")
    Hq, total, D = q.shape
    if cu.ndim != 1 or cu.size < 2 or cu[-1] != total:
        raise ValueError("cu_seqlens must be [n_seq + 1] ending at total")
    o = np.empty((Hq, total, D))
    lse = np.empty((Hq, total))
    rc = lib.attn_varlen_ref_f64(q.ctypes.data, k.ctypes.data, v.ctypes.data, o.ctypes.data,
                                 lse.ctypes.data, cu.ctypes.data, cu.size - 1, Hq, k.shape[0], D,
                                 int(bool(causal)), int(left), int(right), float(scale))
    if rc != 0:
        raise ValueError(f"attn_varlen_ref_f64 failed with code {rc}")
    return o, lse


def e4m3_decode(codes):
    """Values (float64) of e4m3 codes (uint8 array), by the oracle's decode rule."""
    return call_e4m3_decode(_load(), codes)


def call_e4m3_decode(lib, codes):
    c = np.asarray(codes, dtype=np.uint8)
    table = np.array([lib.e4m3_decode(i) for i in range(256)])
    return table[c]


def attn_fp8_ref(q8, k8, v8, descale_q: float, descale_k: float, descale_v: float, causal: bool,
                 scale: float, rows=None, mags=None):
    """Oracle forward on e4m3 inputs: q8 uint8 codes [B, H_q, N, D], k8, v8
    [B, H_kv, N, D]; the tensors are descale_x * value(code).  ``rows``: optional
    int64 flat row ids ((b*H_q + h)*N + i).  ``mags``: optional (w_rel, w_floor),
    then the error-scale sum and its quadrature (rms) counterpart for that
    weight rounding are returned too.

    Returns (o, lse) or (o, lse, mag, rms) as float64, shaped [B, H_q, N, D] and
    [B, H_q, N], or [len(rows), D] and [len(rows)].
    """
    return call_fp8_lib(_load(), q8, k8, v8, descale_q, descale_k, descale_v, causal, scale,
                        rows, mags)


def call_fp8_lib(lib, q8, k8, v8, descale_q, descale_k, descale_v, causal, scale, rows=None,
                 mags=None):
    q8 = np.ascontiguousarray(q8, dtype=np.uint8)
    k8 = np.ascontiguousarray(k8, dtype=np.uint8)
    v8 = np.ascontiguousarray(v8, dtype=np.uint8)
    if q8.ndim != 4 or k8.ndim != 4 or v8.shape != k8.shape:
        raise ValueError("q8 must be [B,H_q,N,D], k8 and v8 [B,H_kv,N,D]")
    B, Hq, N, D = q8.shape
    Hkv = k8.shape[1]
    if k8.shape[0] != B or k8.shape[2] != N or k8.shape[3] != D:
        raise ValueError("shape mismatch between q8 and k8/v8")
    if rows is None:
        o = np.empty((B, Hq, N, D))
        lse = np.empty((B, Hq, N))
        rows_p, n_rows = None, 0
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1)
        o = np.empty((rows.size, D))
        lse = np.empty((rows.size,))
        rows_p, n_rows = rows.ctypes.data, rows.size
    mag = np.empty_like(o) if mags is not None else None
    rms = np.empty_like(o) if mags is not None else None
    w_rel, w_floor = mags if mags is not None else (0.0, 0.0)
    rc = lib.attn_fp8_ref_f64(q8.ctypes.data, k8.ctypes.data, v8.ctypes.data, float(descale_q),
                              float(descale_k), float(descale_v), o.ctypes.data, lse.ctypes.data,
                              None if mag is None else mag.ctypes.data,
                              None if rms is None else rms.ctypes.data, B, Hq, Hkv, N, D,
                              int(bool(causal)), float(scale), float(w_rel), float(w_floor),
                              rows_p, n_rows)
    if rc != 0:
        raise ValueError(f"attn_fp8_ref_f64 failed with code {rc}")
    return (o, lse, mag, rms) if mags is not None else (o, lse)


def attn_blocksparse_ref(q, k, v, kb_ptr, kb_idx, block: int, causal: bool, scale: float,
                         rows=None):
    """Oracle forward with a block-sparse mask: q bf16 bits [B, H_q, N, D], k, v
    [B, H_kv, N, D]; kb_ptr int32 [mask_heads * n_qb + 1] and kb_idx int32 list
    the key blocks (of ``block`` tokens) each query block of each mask head sees
    (mask_heads = 1: shared by all heads).  Rows that see no key get O = 0 and
    LSE = -inf.  Returns (o, lse) as float64, all rows or the flat ``rows``."""
    return call_blocksparse_lib(_load(), q, k, v, kb_ptr, kb_idx, block, causal, scale, rows)


def call_blocksparse_lib(lib, q, k, v, kb_ptr, kb_idx, block, causal, scale, rows=None):
    q = np.ascontiguousarray(q, dtype=np.uint16)
    k = np.ascontiguousarray(k, dtype=np.uint16)
    v = np.ascontiguousarray(v, dtype=np.uint16)
    ptr = np.ascontiguousarray(kb_ptr, dtype=np.int32)
    idx = np.ascontiguousarray(kb_idx, dtype=np.int32)
    if q.ndim != 4 or k.ndim != 4 or v.shape != k.shape:
        raise ValueError("q must be [B,H_q,N,D], k and v [B,H_kv,N,D]")
    B, Hq, N, D = q.shape
    if k.shape[0] != B or k.shape[2] != N or k.shape[3] != D:
        raise ValueError("shape mismatch between q and k/v")
    n_qb = -(-N // int(block))
    if ptr.ndim != 1 or (ptr.size - 1) % n_qb != 0:
        raise ValueError("kb_ptr must hold mask_heads * ceil(N / block) + 1 offsets")
    mask_heads = (ptr.size - 1) // n_qb
    if rows is None:
        o = np.empty((B, Hq, N, D))
        lse = np.empty((B, Hq, N))
        rows_p, n_rows = None, 0
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1)
        o = np.empty((rows.size, D))
        lse = np.empty((rows.size,))
        rows_p, n_rows = rows.ctypes.data, rows.size
    rc = lib.attn_blocksparse_ref_f64(q.ctypes.data, k.ctypes.data, v.ctypes.data, o.ctypes.data,
                                      lse.ctypes.data, ptr.ctypes.data,
                                      idx.ctypes.data if idx.size else None, mask_heads,
                                      int(block), B, Hq, k.shape[1], N, D, int(bool(causal)),
                                      float(scale), rows_p, n_rows)
    if rc != 0:
        raise ValueError(f"attn_blocksparse_ref_f64 failed with code {rc}")
    return o, lse

