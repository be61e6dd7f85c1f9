"""Builds the gfx950 HIP library ``libattn.so`` in-tree with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRCS = [os.path.join(PKG, "csrc", n) for n in
        ("attn_fwd.hip", "attn_fwd_fp8.hip", "attn_bwd.hip", "attn_decode.hip", "status.hip")]
HDR = os.path.join(ROOT, "include", "attn.h")
LIB = os.path.join(PKG, "libattn.so")
ARCH = "gfx950"

# Packed fp32 VALU instructions are disabled for every HIP translation unit.
HIPCC_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Wall", "-Wno-unused-function", "-Wno-inline-asm"]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found: the ROCm toolchain is required to build the library")
    return exe


def build(extra_flags=(), out: str = LIB, verbose: bool = False) -> str:
    """Compile the library (always recompiles).  Returns the .so path."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *HIPCC_FLAGS, *extra_flags, "-I", os.path.join(ROOT, "include"),
           "-o", tmp, *SRCS]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
