"""The C ABI from plain C: tests/c/abi_check.c, compiled with gcc against include/fa.h and linked with
libfa.so and the HIP runtime, runs its argument-check calls (no GPU needed)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def test_c_caller(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    lib_dir = os.path.join(ROOT, "io_aware_exact_18_amd")
    assert os.path.exists(os.path.join(lib_dir, "libfa.so")), "libfa.so is not built"
    exe = str(tmp_path / "abi_check")
    # The HIP runtime headers need the platform macro when compiled by a host compiler.
    cmd = [gcc, "-std=c99", "-O1", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           os.path.join(ROOT, "tests", "c", "abi_check.c"), "-o", exe,
           "-L", lib_dir, "-lfa", "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath," + lib_dir, "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, run.stderr + run.stdout
    assert "all checks passed" in run.stdout
