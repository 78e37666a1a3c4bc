"""Build the native C ABI caller used by tests/test_gpu_native_abi.py:
tests/native/libabi_gpu_check.so, a shared library linked against libzero.so
(rpath to the package directory).  Run after the package build:

    python tests/native/build_native.py
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "zero_sharded_optimizer_reduce_amd")
OUT = os.path.join(HERE, "libabi_gpu_check.so")
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")


def build(verbose: bool = True) -> str:
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O2", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), os.path.join(HERE, "abi_gpu_check.cpp"),
           "-L", PKG, "-lzero", "-Wl,-rpath,$ORIGIN/../../zero_sharded_optimizer_reduce_amd", "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build()
    sys.exit(0)
