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


def _traffic_checked(r, bench):
    """roofline.traffic comes from the committed counter summary exactly when
    the library carries the device code it names."""
    if r["traffic"] is not None:
        assert "not from this run" in r["traffic_source"] and bench.device_code_hash()[:12] in r["traffic_source"]
        assert 0.999 < r["traffic"] / r["algorithmic_bytes_per_launch"] < 1.001
    else:
        assert r["traffic_source"]


def test_chain_runner_line_fields():
    # the default line's own runner at full size (8.03e9 parameters, 112 GB
    # of owner state), a few steps
    import gc

    import torch

    import bench
    print("bench line: zero3_chain_llama8b, 4 steps", flush=True)
    out = bench.run_chain(argparse.Namespace(steps=4, warmup=1, regather_bwd=False))
    gc.collect()
    torch.cuda.empty_cache()
    json.dumps(out)
    assert out["config"]["params"] == 8_029_995_008 and out["config"]["units"] == 34
    assert out["value"] == pytest.approx(out["config"]["params"] / (out["ms_per_step"] * 1e-3))
    k = out["kernels"]
    psi_pad = 32 * k["layer"]["params_padded"] + 2 * k["embedding"]["params_padded"]
    assert out["algorithmic_bytes_per_step"] == 46 * psi_pad
    assert out["memory"]["persistent_bytes_all_owners"] == 14 * psi_pad
    r = out["roofline"]
    assert r["kernel"] == "adam_shard_step" and r["params_per_launch"] == 54_525_952
    assert r["frac"] == pytest.approx(r["achieved"] / bench.PEAK_HBM_GBS)
    _traffic_checked(r, bench)
    # the roofline launch is a quarter of the layer units' 4-launch update
    # span; the breakdown takes one event gap off that span, and adds up to
    # about the step
    assert r["launch_ms"] == pytest.approx(k["layer"]["adam_shard_step"]["ms"] + k["event_overhead_ms"] / 4)
    assert k["sum_ms"] == pytest.approx(out["ms_per_step"], rel=0.05)
    assert out["fused_variant"]["ms_per_step"] < out["ms_per_step"]


def test_owner_share_runner_line_fields():
    import gc

    import torch

    import bench
    print("bench line: owner_share_8b_buckets, 4 steps", flush=True)
    out = bench.run_owner_share(argparse.Namespace(steps=4, warmup=1, regather_bwd=False))
    gc.collect()
    torch.cuda.empty_cache()
    json.dumps(out)
    assert out["config"]["params"] == 2_000_000_000 and out["config"]["buckets"] == 30
    r = out["roofline"]
    assert r["params_per_launch"] == 1 << 26
    _traffic_checked(r, bench)
    assert out["fused_variant"]["ms_per_step"] < out["ms_per_step"]
