"""The C-ABI library on the host: it loads, exports every declared symbol and
rejects bad arguments before touching the GPU (CPU only; no kernel launch)."""
import ctypes
import math
import os
import re
import subprocess

import pytest

import scaled_dot_product_17_amd as sdpa
from scaled_dot_product_17_amd import _build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sdpa.LIB_PATH):
        _build.build()
    return sdpa.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\([^;{]*\)\s*;", text)))


def test_header_declares_the_exports():
    assert declared_functions() == sorted(sdpa.EXPORTED)


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", sdpa.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    syms = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    for name in declared_functions():
        assert name in syms, f"{name} not exported"
        assert hasattr(lib, name)


def test_status_strings(lib):
    for code, name in sdpa.STATUS_NAMES.items():
        s = sdpa.status_string(code)
        assert isinstance(s, str) and s and s != "unknown status", name
    assert sdpa.status_string(12345) == "unknown status"


def test_flops_convention(lib):
    assert sdpa.attn_fwd_flops(2, 16, 16384, 128, False) == 4.0 * 2 * 16 * 16384 ** 2 * 128
    assert sdpa.attn_fwd_flops(2, 16, 16384, 128, True) == 2.0 * 2 * 16 * 16384 ** 2 * 128


# Fake, 256-byte aligned and far-apart addresses: never dereferenced because
# every call below fails validation before any HIP call.
Q, K, V, O, L = 0x100000, 0x200000000, 0x400000000, 0x600000000, 0x800000000
OK_ARGS = dict(q=Q, k=K, v=V, o=O, lse=L, B=1, H_q=4, H_kv=2, N=64, D=128, causal=0,
               scale=1 / math.sqrt(128), stream=None)


def call(**kw):
    a = dict(OK_ARGS)
    a.update(kw)
    return sdpa.attn_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H_q"], a["H_kv"],
                         a["N"], a["D"], a["causal"], a["scale"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(k=None), 1), (dict(v=None), 1), (dict(o=None), 1),
    (dict(B=0), 2), (dict(H_q=-1), 2), (dict(H_kv=0), 2), (dict(N=0), 2), (dict(D=0), 2),
    (dict(N=1 << 23), 2),
    (dict(H_q=3, H_kv=2), 3),
    (dict(D=64), 4), (dict(D=256), 4),
    (dict(scale=float("nan")), 5), (dict(scale=float("inf")), 5), (dict(scale=-float("inf")), 5),
    (dict(q=Q + 8), 6), (dict(o=O + 2), 6), (dict(lse=L + 2), 6),
    (dict(o=Q), 7), (dict(o=K + 4096), 7), (dict(lse=O + 64), 7), (dict(lse=V), 7),
])
def test_argument_errors(lib, kw, code):
    assert call(**kw) == code


def test_valid_arguments_without_gpu_report_device(lib):
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present: this case would launch on fake pointers")
    assert call() == 9


def test_python_binding_rejects_bad_tensors():
    import torch
    q = torch.zeros(1, 2, 8, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        sdpa.fwd(q, q, q)                       # CPU tensors
    with pytest.raises(ValueError):
        sdpa.fwd(q.float(), q, q)               # wrong dtype
    with pytest.raises(ValueError):
        sdpa.fwd(q[..., :64], q, q)             # 3-D / shape checks happen first


def test_faithful_rounding_helper():
    """Both bf16 values bracketing x are accepted, nothing farther is."""
    import numpy as np
    from synth import bf16_bits_to_f32
    from tests.parity import faithful
    rng = np.random.default_rng(0)
    ref = rng.standard_normal(20000) * 5
    grid = bf16_bits_to_f32(np.arange(0, 0x7F80, dtype=np.uint16)).astype(np.float64)
    grid = np.unique(np.concatenate([grid, -grid]))
    i = np.searchsorted(grid, ref)
    lo, hi, far = grid[i - 1], grid[i], grid[i - 2]
    assert faithful(lo, ref).all() and faithful(hi, ref).all()
    assert not faithful(far, ref).any()


def test_bwd_flops_convention(lib):
    assert sdpa.attn_bwd_flops(2, 16, 16384, 128, False) == 10.0 * 2 * 16 * 16384 ** 2 * 128
    assert sdpa.attn_bwd_flops(2, 16, 16384, 128, True) == 5.0 * 2 * 16 * 16384 ** 2 * 128


# attn_bwd: inputs q, k, v, o, dout, lse; outputs dq, dk, dv, delta (fake, far apart)
BW = dict(q=0x100000, k=0x200000000, v=0x400000000, o=0x600000000, dout=0x800000000,
          lse=0xA00000000, dq=0xC00000000, dk=0xE00000000, dv=0x1000000000,
          delta=0x1200000000, B=1, H_q=4, H_kv=2, N=64, D=128, causal=1,
          scale=1 / math.sqrt(128), stream=None)


def call_bwd(**kw):
    a = dict(BW)
    a.update(kw)
    return sdpa.attn_bwd(a["q"], a["k"], a["v"], a["o"], a["dout"], a["lse"], a["dq"], a["dk"],
                         a["dv"], a["delta"], a["B"], a["H_q"], a["H_kv"], a["N"], a["D"],
                         a["causal"], a["scale"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(o=None), 1), (dict(dout=None), 1), (dict(lse=None), 1),
    (dict(dq=None), 1), (dict(dk=None), 1), (dict(dv=None), 1), (dict(delta=None), 1),
    (dict(B=0), 2), (dict(N=-3), 2), (dict(N=1 << 23), 2),
    (dict(H_q=6, H_kv=4), 3), (dict(D=64), 4),
    (dict(scale=float("nan")), 5),
    (dict(dout=0x800000008), 6), (dict(dk=0xE00000002), 6), (dict(delta=0x1200000002), 6),
    (dict(dq=0x100000), 7), (dict(dk=0x400000000 + 256), 7), (dict(delta=0x600000000), 7),
    (dict(dv=0xC00000000 + 1024), 7), (dict(delta=0xA00000000 + 64), 7),
])
def test_bwd_argument_errors(lib, kw, code):
    assert call_bwd(**kw) == code


def test_bwd_valid_arguments_without_gpu_report_device(lib):
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present: this case would launch on fake pointers")
    assert call_bwd() == 9


def test_python_bwd_rejects_bad_tensors():
    import torch
    q = torch.zeros(1, 2, 8, 128, dtype=torch.bfloat16)
    lse = torch.zeros(1, 2, 8)
    with pytest.raises(ValueError):
        sdpa.bwd(q, q, q, q, lse, q)            # CPU tensors


def call_dq(**kw):
    a = dict(BW)
    a.update(kw)
    return sdpa.attn_bwd_dq(a["q"], a["k"], a["v"], a["o"], a["dout"], a["lse"], a["dq"],
                            a["delta"], a["B"], a["H_q"], a["H_kv"], a["N"], a["D"], a["causal"],
                            a["scale"], a["stream"])


def call_dkdv(**kw):
    a = dict(BW)
    a.update(kw)
    return sdpa.attn_bwd_dkdv(a["q"], a["k"], a["v"], a["dout"], a["lse"], a["delta"], a["dk"],
                              a["dv"], a["B"], a["H_q"], a["H_kv"], a["N"], a["D"], a["causal"],
                              a["scale"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(o=None), 1), (dict(dq=None), 1), (dict(delta=None), 1), (dict(N=0), 2),
    (dict(H_q=5), 3), (dict(D=96), 4), (dict(scale=float("inf")), 5), (dict(dq=0xC00000004), 6),
    (dict(delta=0xA00000000), 7), (dict(dq=0x600000000 + 512), 7),
])
def test_bwd_dq_argument_errors(lib, kw, code):
    assert call_dq(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(delta=None), 1), (dict(dk=None), 1), (dict(k=None), 1), (dict(B=-1), 2),
    (dict(H_kv=3), 3), (dict(D=129), 4), (dict(delta=0x1200000001), 6),
    (dict(dk=0x1200000000), 7), (dict(dv=0xE00000000 + 16), 7), (dict(dv=0x800000000), 7),
])
def test_bwd_dkdv_argument_errors(lib, kw, code):
    assert call_dkdv(**kw) == code


def test_bwd_split_calls_without_gpu_report_device(lib):
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present: this case would launch on fake pointers")
    assert call_dq() == 9 and call_dkdv() == 9
