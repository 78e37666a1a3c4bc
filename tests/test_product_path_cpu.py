"""The product path has no fallback: without libzero.so every call raises, and
nothing in the package, its C sources or the drivers imports or links the
oracle (which is test infrastructure only)."""
import ast
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "zero_sharded_optimizer_reduce_amd")


def test_missing_library_raises_in_every_entry_point():
    code = r"""
import os, sys
sys.path.insert(0, sys.argv[1])
import numpy as np, torch
from zero_sharded_optimizer_reduce_amd import _lib
_lib.LIB_PATH = os.path.join(sys.argv[1], "no_such_dir", "libzero.so")
import zero_sharded_optimizer_reduce_amd.api as z
calls = [
    lambda: z.zero_rank_weights(None, 4),
    lambda: z.zero_shard_layout([1000], 4),
    lambda: z.zero_adam_scalars_compute(dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, step=1)),
]
for f in calls:
    try:
        f()
    except RuntimeError as e:
        assert "no CPU fallback" in str(e), e
    else:
        raise SystemExit("a call succeeded without the library")
print("ok")
"""
    r = subprocess.run([sys.executable, "-c", code, ROOT], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr


def _python_imports(path):
    tree = ast.parse(open(path, encoding="utf-8").read(), path)
    names = set()
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            names.update(a.name.split(".")[0] for a in node.names)
        elif isinstance(node, ast.ImportFrom) and node.level == 0 and node.module:
            names.add(node.module.split(".")[0])
    return names


def test_package_never_imports_the_oracle():
    for dirpath, _, files in os.walk(PKG):
        for f in files:
            path = os.path.join(dirpath, f)
            if f.endswith(".py"):
                assert "oracle" not in _python_imports(path), path
            elif f.endswith((".hip", ".cpp", ".h")):
                text = open(path, encoding="utf-8").read()
                assert "oracle/" not in text and "zero_oracle" not in text, path
