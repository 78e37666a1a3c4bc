"""The benchmark's command-line contract on the CPU: more than one GPU is
refused with a message, and the oracle baseline reports its fields."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_cpu_baseline_fields():
    sys.path.insert(0, ROOT)
    import bench
    out = bench.cpu_baseline(0.2)
    json.dumps(out)
    assert out["kind"] == "oracle" and out["unit"] == "params/s"
    assert out["value"] > 0 and out["cores"] >= 1
    assert out["single_thread"]["cores"] == 1 and out["single_thread"]["value"] > 0
    assert "2^22" in out["sample"]


def test_timed_regions_run_without_the_cyclic_collector():
    # a full collection inside a timed loop stalls the launching thread long
    # enough for the GPU to run dry; the region turns it off and restores it
    import gc

    import bench
    assert gc.isenabled()
    with bench.no_gc():
        assert not gc.isenabled()
    assert gc.isenabled()
    try:
        with bench.no_gc():
            raise RuntimeError("inside")
    except RuntimeError:
        pass
    assert gc.isenabled()
    gc.disable()
    try:
        with bench.no_gc():
            assert not gc.isenabled()
        assert not gc.isenabled()      # a caller's own setting is kept
    finally:
        gc.enable()
