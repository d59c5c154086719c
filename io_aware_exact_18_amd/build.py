"""Build libfa.so (the gfx950 attention library) in-tree with hipcc.

Usage: python -m io_aware_exact_18_amd.build   (or call ``build()``).  Compiles every source under
``csrc/`` for gfx950 into objects under ``_build/`` in parallel, then links
``io_aware_exact_18_amd/libfa.so``.  No GPU is needed: hipcc cross-compiles.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libfa.so")
ARCH = "gfx950"

SOURCES = ["fa_api.hip", "fa_fwd.hip", "fa_bwd.hip", "fa_fwd_fp8.hip", "fa_decode.hip",
           "fa_bwd_fp8.hip"]

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-mcode-object-version=5",
    "-munsafe-fp-atomics",
    # Packed fp32 VALU forms are kept out of the generated code on purpose.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the library cannot be built")
    return path


def _compile(src, extra):
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        err = "\n".join(l for l in r.stderr.splitlines() if "error" in l)[:4000]
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{err or r.stderr[-4000:]}")
    return obj, r.stderr


def build(verbose=False, extra_flags=()):
    """Compile and link libfa.so; returns its path.  Raises RuntimeError on any compiler error."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        results = list(ex.map(lambda s: _compile(s, list(extra_flags)), SOURCES))
    objs = [o for o, _ in results]
    if verbose:
        for _, err in results:
            if err.strip():
                print(err, file=sys.stderr)
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


PROBE_SRC = os.path.join(ROOT, "tests", "hip", "fa_probe.hip")
PROBE_LIB = os.path.join(ROOT, "tests", "hip", "libfa_probe.so")


def build_probe():
    """Compile the tests' conversion probe (tests/hip/fa_probe.hip, not part of libfa.so) into
    tests/hip/libfa_probe.so with the library's flags; returns its path."""
    tmp = PROBE_LIB + ".tmp"
    cmd = [hipcc(), *COMMON_FLAGS, "-shared", PROBE_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for the probe:\n{' '.join(cmd)}\n{r.stderr[-4000:]}")
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    print(build_probe())
