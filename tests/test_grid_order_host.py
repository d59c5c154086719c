"""The grid-order functions of the tiled kernels on the host: tests/c/grid_order_check.cpp includes
the library's own device header (fa_common.h, fa_launch.h), compiled by hipcc for the host only, and
checks xcd_remap and head_tile on 13,614 grids (1–72 heads, 1–100 tiles, one to three resident
workgroups per compute unit, plain and XCD order): both are bijections, each head's tiles start in
order, a head stays within one XCD's eighth of the items, and grouped heads alternate tile by tile.
No GPU needed."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def test_grid_order_host(tmp_path):
    hipcc = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "grid_order_check")
    cmd = [hipcc, "-x", "hip", "--offload-host-only", "-O2", "-std=c++17", "-Wall", "-Werror",
           "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "io_aware_exact_18_amd", "csrc"),
           os.path.join(ROOT, "tests", "c", "grid_order_check.cpp"), "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "all checks passed" in run.stdout
