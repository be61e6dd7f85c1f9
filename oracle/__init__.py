"""fp64 CPU oracle for the attention forward pass.

TEST INFRASTRUCTURE ONLY: used by ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py``.  The product library never imports,
links or calls anything here, and nothing here imports the product package.

``attn_ref`` wraps the C routine in ``attn_ref.c`` (the plain definition,
softmax(scale * Q K^T [causal]) V and its log-sum-exp, in double precision).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_ref.c")
_LIB = os.path.join(_HERE, "libattn_ref.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with the host C compiler (no fast-math: IEEE double)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-fno-fast-math",
               "-ffp-contract=off", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _bind(path: str):
    lib = ctypes.CDLL(path)
    fn = lib.attn_ref_f64
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 6 + [
        ctypes.c_double, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64]
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
