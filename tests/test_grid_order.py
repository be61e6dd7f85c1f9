"""The dealt grid order of the forward kernels, checked on the host: the
header's order functions are compiled into a small host program
(grid_order_main.hip) that walks every workgroup id of each launch shape."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "scaled_dot_product_17_amd", "csrc")


def test_dealt_order_covers_every_tile_once(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not found")
    exe = str(tmp_path / "grid_order")
    res = subprocess.run([hipcc, "-O2", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature",
                          "-Xclang", "-packed-fp32-ops", "-w", "-I", CSRC,
                          "-o", exe, os.path.join(HERE, "grid_order_main.hip")],
                         capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stdout + res.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    assert run.returncode == 0 and run.stdout.startswith("ok"), run.stdout + run.stderr
    print(run.stdout.strip())
