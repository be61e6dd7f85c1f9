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


def test_bwd_splits_and_workspace_bytes(lib):
    # MQA, B = 8, N = 2048: 128 dK/dV workgroups -> 2 parts reach 256
    assert sdpa.attn_bwd_splits(8, 16, 1, 2048, 128) == 2
    assert sdpa.attn_bwd_workspace_bytes(8, 16, 1, 2048, 128) == 2 * 2 * 8 * 2048 * 128 * 4
    # the grid already has 256 workgroups: no split, no workspace
    assert sdpa.attn_bwd_splits(8, 16, 2, 2048, 128) == 1
    assert sdpa.attn_bwd_workspace_bytes(8, 16, 2, 2048, 128) == 0
    assert sdpa.attn_bwd_splits(2, 16, 16, 16384, 128) == 1
    # tiny grid: the largest divisor of the group up to 16
    assert sdpa.attn_bwd_splits(1, 16, 1, 512, 128) == 16
    assert sdpa.attn_bwd_splits(1, 12, 1, 512, 128) == 12
    assert sdpa.attn_bwd_splits(1, 4, 2, 256, 128) == 2
    # causal: four workgroups per CU, eight from N = 8192 (a causal key tile's
    # work falls with its index)
    assert sdpa.attn_bwd_splits(1, 16, 1, 32768, 128) == 1
    assert sdpa.attn_bwd_splits(1, 16, 1, 32768, 128, causal=True) == 8
    assert sdpa.attn_bwd_splits(2, 16, 2, 8192, 128, causal=True) == 8
    assert sdpa.attn_bwd_splits(8, 16, 2, 2048, 128, causal=True) == 4
    assert sdpa.attn_bwd_splits(8, 16, 1, 2048, 128, causal=True) == 8
    assert sdpa.attn_bwd_splits(2, 16, 16, 16384, 128, causal=True) == 1
    assert sdpa.attn_bwd_workspace_bytes(1, 16, 1, 32768, 128, True) == 8 * 2 * 32768 * 128 * 4
    # requested: the largest divisor of the group not above the request
    assert sdpa.attn_bwd_splits(8, 16, 1, 2048, 128, n_splits=3) == 2
    assert sdpa.attn_bwd_splits(1, 12, 1, 512, 128, n_splits=5) == 4
    assert sdpa.attn_bwd_splits(1, 12, 1, 512, 128, True, 5) == 4
    assert sdpa.attn_bwd_splits(1, 12, 1, 512, 128, n_splits=1) == 1
    assert sdpa.attn_bwd_workspace_bytes(1, 12, 1, 512, 128, n_splits=5) == 4 * 2 * 512 * 128 * 4
    # invalid arguments -> 0
    assert sdpa.attn_bwd_splits(8, 15, 2, 2048, 128) == 0
    assert sdpa.attn_bwd_splits(8, 16, 1, 2048, 64) == 0
    assert sdpa.attn_bwd_splits(0, 16, 1, 2048, 128) == 0
    assert sdpa.attn_bwd_workspace_bytes(8, 16, 1, 0, 128) == 0


# attn_bwd_ws on a shape that splits (MQA, 4 query heads, 2 parts requested)
BWS = dict(BW, H_q=4, H_kv=1, n_splits=2, ws=0x1400000000, ws_bytes=1 << 30)


def call_bwd_ws(**kw):
    a = dict(BWS)
    a.update(kw)
    return sdpa.attn_bwd_ws(a["q"], a["k"], a["v"], a["o"], a["dout"], a["lse"], a["dq"], a["dk"],
                            a["dv"], a["delta"], a["B"], a["H_q"], a["H_kv"], a["N"], a["D"],
                            a["causal"], a["scale"], a["n_splits"], a["ws"], a["ws_bytes"],
                            a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(ws=None), 1), (dict(q=None), 1), (dict(N=0), 2), (dict(H_q=5, H_kv=2), 3), (dict(D=64), 4),
    (dict(scale=float("nan")), 5), (dict(ws=0x1400000008), 6),
    (dict(ws=0x100000), 7), (dict(ws=0x1200000000), 7), (dict(dk=0x1400000000 + 4096), 7),
    (dict(ws_bytes=2 * 2 * 64 * 128 * 4 - 16), 10), (dict(ws_bytes=0), 10),
])
def test_bwd_ws_argument_errors(lib, kw, code):
    assert call_bwd_ws(**kw) == code


def test_bwd_ws_valid_arguments_without_gpu_report_device(lib):
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present: this case would launch on fake pointers")
    assert call_bwd_ws() == 9
    assert call_bwd_ws(ws_bytes=2 * 2 * 64 * 128 * 4) == 9      # exactly enough
    assert call_bwd_ws(n_splits=1, ws=None, ws_bytes=0) == 9     # one part: attn_bwd, no workspace


# attn_decode / attn_lse_merge (fake, far-apart addresses; validation only)
DC = dict(q=0x100000, k=0x200000000, v=0x400000000, o=0x600000000, lse=0x800000000, B=8,
          H_q=16, H_kv=2, M=1, L=32768, D=128, causal=0, scale=1 / math.sqrt(128), n_splits=0,
          ws=0xA00000000, ws_bytes=1 << 30, stream=None)


def call_dec(**kw):
    a = dict(DC)
    a.update(kw)
    return sdpa.attn_decode(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H_q"], a["H_kv"],
                            a["M"], a["L"], a["D"], a["causal"], a["scale"], a["n_splits"], a["ws"],
                            a["ws_bytes"], a["stream"])


def test_decode_workspace_bytes(lib):
    # 16 K/V heads x 1 column block -> 64 splits of 512 keys; partial O and LSE
    # of 128 rows: 128*64*128*4 bytes, then 128*64*4 bytes at a 256-byte boundary
    assert sdpa.attn_decode_workspace_bytes(8, 16, 2, 1, 32768, 128) == 128 * 64 * 128 * 4 + 128 * 64 * 4
    # explicit split count; capped at one split per 32-key block
    assert sdpa.attn_decode_workspace_bytes(1, 4, 1, 2, 1000, 128, 7) == 8 * 7 * 128 * 4 + 8 * 7 * 4
    assert sdpa.attn_decode_workspace_bytes(1, 4, 1, 2, 40, 128, 50) == 8 * 2 * 128 * 4 + 8 * 2 * 4
    assert sdpa.attn_decode_workspace_bytes(1, 3, 2, 1, 40, 128) == 0   # invalid -> 0
    assert sdpa.attn_decode_splits(8, 16, 2, 1, 32768, 128) == 64
    assert sdpa.attn_decode_splits(1, 16, 1, 1, 32768, 128) == 256   # L / (8 g M) cap
    assert sdpa.attn_decode_splits(1, 4, 1, 2, 1000, 128, 7) == 7
    assert sdpa.attn_decode_splits(1, 4, 1, 2, 40, 128, 50) == 2
    assert sdpa.attn_decode_splits(1, 4, 1, 2, 40, 64, 5) == 0
    assert sdpa.attn_decode_flops(2, 4, 3, 10, 128, False) == 4.0 * 2 * 4 * 128 * 30
    assert sdpa.attn_decode_flops(2, 4, 3, 10, 128, True) == 4.0 * 2 * 4 * 128 * (8 + 9 + 10)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(ws=None), 1), (dict(o=None), 1),
    (dict(M=0), 2), (dict(L=0), 2), (dict(causal=1, M=5, L=4), 2), (dict(L=1 << 23), 2),
    (dict(H_q=15), 3), (dict(D=64), 4), (dict(scale=float("nan")), 5),
    (dict(k=0x200000008), 6), (dict(ws=0xA00000004), 6), (dict(lse=0x800000002), 6),
    (dict(o=0x100000 + 64), 7), (dict(ws=0x400000000 + 4096), 7), (dict(lse=0x600000000 + 32), 7),
    (dict(ws_bytes=1000), 10),
])
def test_decode_argument_errors(lib, kw, code):
    assert call_dec(**kw) == code


def call_dec_noalloc(**kw):
    a = dict(DC)
    a.update(kw)
    return sdpa.attn_decode_noalloc(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H_q"],
                                    a["H_kv"], a["M"], a["L"], a["D"], a["causal"], a["scale"],
                                    a["n_splits"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(o=None), 1),
    (dict(M=0), 2), (dict(causal=1, M=5, L=4), 2), (dict(H_q=15), 3), (dict(D=64), 4),
    (dict(scale=float("inf")), 5), (dict(k=0x200000008), 6), (dict(lse=0x800000002), 6),
    (dict(o=0x100000 + 64), 7), (dict(lse=0x600000000 + 32), 7),
    # partial results beyond the fixed scratch array: 2048 rows x 32 splits x 516 B
    (dict(H_kv=16, M=16, n_splits=32), 11),
])
def test_decode_noalloc_argument_errors(lib, kw, code):
    assert call_dec_noalloc(**kw) == code


def test_decode_noalloc_scratch_size(lib):
    assert sdpa.DECODE_SCRATCH_BYTES == 16 << 20
    text = open(HEADER).read()
    assert "#define ATTN_DECODE_SCRATCH_BYTES ((size_t)16 << 20)" in text
    # the largest split count that fits is accepted by the size check (it then
    # reports the missing device), one more split is refused
    fits = sdpa.attn_decode_workspace_bytes(8, 16, 16, 16, 32768, 128, 15)
    over = sdpa.attn_decode_workspace_bytes(8, 16, 16, 16, 32768, 128, 16)
    assert fits <= sdpa.DECODE_SCRATCH_BYTES < over
    assert call_dec_noalloc(H_kv=16, M=16, n_splits=16) == 11


def test_decode_valid_arguments_without_gpu_report_device(lib):
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present: this case would launch on fake pointers")
    assert call_dec() == 9 and call_dec(lse=None) == 9
    assert call_dec_noalloc() == 9 and call_dec_noalloc(lse=None) == 9


@pytest.mark.parametrize("args,code", [
    ((None, 0x200000000, 10, 4, 128, 0x400000000, 0x600000000), 1),
    ((0x100000, 0x200000000, -1, 4, 128, 0x400000000, 0x600000000), 2),
    ((0x100000, 0x200000000, 10, 0, 128, 0x400000000, 0x600000000), 2),
    ((0x100000, 0x200000000, 10, 4, 64, 0x400000000, 0x600000000), 4),
    ((0x100008, 0x200000000, 10, 4, 128, 0x400000000, 0x600000000), 6),
    ((0x100000, 0x200000000, 10, 4, 128, 0x100000 + 256, 0x600000000), 7),
    ((0x100000, 0x200000000, 10, 4, 128, 0x400000000, 0x400000000 + 8), 7),
])
def test_lse_merge_argument_errors(lib, args, code):
    assert sdpa.attn_lse_merge(*args, None) == code


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(op=None), 1), (dict(n_splits=0), 2), (dict(n_splits=1025), 2),
    (dict(M=0), 2), (dict(H_kv=3), 3), (dict(D=96), 4), (dict(op=0x600000004), 6),
    (dict(op=0x200000000 + 512), 7), (dict(lp=0x600000000 + 128), 7),
])
def test_decode_partial_argument_errors(lib, kw, code):
    a = dict(q=0x100000, k=0x200000000, v=0x400000000, op=0x600000000, lp=0x800000000, B=8,
             H_q=16, H_kv=2, M=1, L=32768, D=128, causal=0, scale=0.1, n_splits=7)
    a.update(kw)
    assert sdpa.attn_decode_partial(a["q"], a["k"], a["v"], a["op"], a["lp"], a["B"], a["H_q"],
                                    a["H_kv"], a["M"], a["L"], a["D"], a["causal"], a["scale"],
                                    a["n_splits"], None) == code


# attn_fwd_varlen (fake, far-apart addresses; validation only)
VL = dict(q=0x100000, k=0x200000000, v=0x400000000, o=0x600000000, lse=0x800000000,
          cu=0xA00000000, n_seq=4, max_seqlen=1000, total=3000, H_q=8, H_kv=2, D=128, causal=1,
          left=-1, right=-1, scale=0.1, stream=None)


def call_varlen(**kw):
    a = dict(VL)
    a.update(kw)
    return sdpa.attn_fwd_varlen(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cu"], a["n_seq"],
                                a["max_seqlen"], a["total"], a["H_q"], a["H_kv"], a["D"],
                                a["causal"], a["left"], a["right"], a["scale"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(cu=None), 1), (dict(q=None), 1), (dict(n_seq=0), 2), (dict(max_seqlen=0), 2),
    (dict(total=0), 2), (dict(total=1 << 23), 2), (dict(H_q=7), 3), (dict(D=64), 4),
    (dict(scale=float("inf")), 5), (dict(cu=0xA00000002), 6), (dict(v=0x400000008), 6),
    (dict(o=0xA00000000 - 64), 7), (dict(lse=0x100000 + 128), 7), (dict(lse=0x600000000 + 16), 7),
])
def test_varlen_argument_errors(lib, kw, code):
    assert call_varlen(**kw) == code


def test_varlen_valid_arguments_without_gpu_report_device(lib):
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present: this case would launch on fake pointers")
    assert call_varlen() == 9 and call_varlen(left=100, right=0, lse=None) == 9


# attn_fwd_fp8 (fake, far-apart addresses; validation only)
F8 = dict(OK_ARGS, dq=0.02, dk=0.03, dv=0.5)


def call_fp8(**kw):
    a = dict(F8)
    a.update(kw)
    return sdpa.attn_fwd_fp8(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H_q"],
                             a["H_kv"], a["N"], a["D"], a["causal"], a["scale"], a["dq"], a["dk"],
                             a["dv"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(v=None), 1), (dict(o=None), 1),
    (dict(B=0), 2), (dict(N=0), 2), (dict(N=1 << 23), 2), (dict(H_q=3, H_kv=2), 3),
    (dict(D=64), 4),
    (dict(scale=float("nan")), 5), (dict(dq=float("inf")), 5), (dict(dk=float("nan")), 5),
    (dict(dv=float("-inf")), 5), (dict(scale=1e30, dq=1e30), 5),
    (dict(q=Q + 8), 6), (dict(k=K + 1), 6), (dict(o=O + 2), 6), (dict(lse=L + 2), 6),
    (dict(o=Q), 7), (dict(o=K + 4096), 7), (dict(lse=O + 64), 7), (dict(lse=V), 7),
    (dict(lse=O + 65536 - 4), 7),
])
def test_fp8_argument_errors(lib, kw, code):
    assert call_fp8(**kw) == code


def test_fp8_valid_arguments_without_gpu_report_device(lib):
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present: this case would launch on fake pointers")
    assert call_fp8() == 9 and call_fp8(lse=None, causal=1, scale=-0.1) == 9
    assert call_fp8(lse=O + 65536) == 9   # o is 2 bytes per element: just past its end


def test_python_fp8_rejects_bad_tensors():
    import torch
    q = torch.zeros(1, 2, 8, 128, dtype=torch.uint8)
    with pytest.raises(ValueError):
        sdpa.fwd_fp8(q, q, q)                       # CPU tensors
    with pytest.raises(ValueError):
        sdpa.fwd_fp8(q.to(torch.bfloat16), q, q)    # wrong dtype


# attn_fwd_blocksparse (fake, far-apart addresses; validation only).  N = 64 -> one
# 128-block: kb_ptr holds 2 offsets (mask_heads = 1).
BS = dict(OK_ARGS, ptr=0xA00000000, idx=0xC00000000, nnz=1, mh=1)


def call_bs(**kw):
    a = dict(BS)
    a.update(kw)
    return sdpa.attn_fwd_blocksparse(a["q"], a["k"], a["v"], a["o"], a["lse"], a["ptr"], a["idx"],
                                     a["nnz"], a["mh"], a["B"], a["H_q"], a["H_kv"], a["N"],
                                     a["D"], a["causal"], a["scale"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(ptr=None), 1), (dict(idx=None), 1), (dict(q=None), 1),
    (dict(nnz=-1), 2), (dict(mh=2), 2), (dict(N=0), 2), (dict(N=2048 * 128 + 1), 2),
    (dict(H_q=3), 3), (dict(D=64), 4), (dict(scale=float("nan")), 5),
    (dict(ptr=0xA00000002), 6), (dict(idx=0xC00000001), 6), (dict(q=Q + 8), 6),
    (dict(o=0xA00000000 - 64), 7), (dict(lse=0xC00000000), 7), (dict(o=K), 7),
])
def test_blocksparse_argument_errors(lib, kw, code):
    assert call_bs(**kw) == code


def test_blocksparse_valid_arguments_without_gpu_report_device(lib):
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present: this case would launch on fake pointers")
    assert call_bs() == 9 and call_bs(idx=None, nnz=0, causal=1) == 9
    assert call_bs(mh=4, N=256) == 9
