"""The benchmark's JSON line on the GPU, in this process: the flat-unit runner
on the 2^20-parameter tensor (the same code path as the 7B-class layer's)
returns every field of the line's contract, a roofline entry against the
8 TB/s peak and consistent step figures."""
import argparse
import json
import os
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def test_flat_runner_line_fields():
    import bench
    print("bench line: tiny_flat_1m, 4 steps", flush=True)
    out = bench.run_tiny(argparse.Namespace(steps=4, warmup=1, regather_bwd=False))
    json.dumps(out)
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "kernels", "fused_variant"):
        assert key in out, key
    assert out["metric"] == bench.METRIC and out["unit"] == "params/s" and out["n_gpus"] == 1
    assert out["steps"] == 4 and out["warmup"] == 1 and out["higher_is_better"] is True
    assert out["value"] == pytest.approx(out["config"]["params"] / (out["ms_per_step"] * 1e-3))
    r = out["roofline"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == bench.PEAK_HBM_GBS
    assert r["achieved"] > 0 and r["frac"] == pytest.approx(r["achieved"] / r["peak"])
    assert r["algorithmic_bytes_per_launch"] == bench.B_ADAM * r["params_per_launch"]
    k = out["kernels"]
    assert k["reduce_scatter"]["ms"] > 0 and k["adam_shard_step"]["ms"] > 0 and k["all_gather"]["ms"] > 0
    assert out["fused_variant"]["ms_per_step"] > 0
