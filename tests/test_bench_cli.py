"""The benchmark's command-line contract on the CPU: more than one GPU is
refused with a message, the default workload is the 8B ZeRO-3 chain, and the
oracle baseline reports its fields and its extrapolation."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


@pytest.mark.parametrize("kind, psi", [("zero3_chain_llama8b", 8_029_995_008),
                                       ("layer7b_weighted_adamw", 202_375_168),
                                       ("owner_share_8b_buckets", 2_000_000_000),
                                       ("offload_owner_8b_two_slots", 2_000_000_000)])
def test_cpu_baseline_fields(kind, psi):
    sys.path.insert(0, ROOT)
    import bench
    out = bench.cpu_baseline(kind, 0.2)
    json.dumps(out)
    assert out["kind"] == "oracle" and out["unit"] == "params/s"
    assert out["value"] > 0 and out["cores"] >= 1
    assert out["single_thread"]["cores"] == 1 and out["single_thread"]["value"] > 0
    assert "2^22" in out["sample"] and f"{psi:,}" in out["sample"]
    # the extrapolation to a whole step is the parameter count over the rate
    assert out["extrapolated_step_s"] == pytest.approx(psi / out["value"])


def test_default_workload_is_the_largest_single_gpu_config():
    import bench
    src = open(os.path.join(ROOT, "bench.py")).read()
    assert 'ap.add_argument("--workload", default="zero3_chain_llama8b"' in src
    assert "zero3_chain_llama8b" in bench.CPU_SAMPLES and "zero3_chain_llama8b" in bench.RUNNERS


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


def test_stored_traffic_is_used_only_for_the_device_code_it_measured(tmp_path, monkeypatch, libzero):
    import bench
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    code = bench.device_code_hash()
    assert len(code) == 64 and code == bench.device_code_hash()
    f = tmp_path / "kern_work_traffic.txt"
    f.write_text(f"# comment: ignored\ndevice_code_sha256: {code}\nparams_per_launch: 100\n"
                 "hbm_bytes_per_launch: 3000\n")
    value, source = bench._traffic("kern", "work", 100)
    assert value == 3000.0 and code[:12] in source and "not from this run" in source
    assert bench._traffic("kern", "work", 99)[0] is None                 # another launch size
    assert bench._traffic("other", "work", 100)[0] is None               # no summary
    f.write_text(f"device_code_sha256: {'0' * 64}\nparams_per_launch: 100\nhbm_bytes_per_launch: 3000\n")
    value, source = bench._traffic("kern", "work", 100)
    assert value is None and "other device code" in source
    with pytest.raises(ValueError):
        bench._elf_section(__file__, ".hip_fatbin")                      # not an ELF file


def test_child_workload_failure_is_reported_not_raised():
    # without a GPU the child exits with an error; the line records it
    import argparse

    import bench
    out = bench._child_workload("layer7b_weighted_adamw", argparse.Namespace(steps=1, warmup=0))
    assert "error" in out and "exited with 1" in out["error"]


def test_committed_traffic_summaries_match_the_built_device_code(libzero):
    # the bench line reports roofline.traffic from these files only while the
    # library carries the machine code their counters were taken on: a kernel
    # change without new counter passes would turn the field into null
    import glob

    import bench
    code = bench.device_code_hash()
    files = sorted(glob.glob(os.path.join(ROOT, "profiles", "*_traffic.txt")))
    assert files
    for path in files:
        kv = {}
        for line in open(path):
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
        assert kv["device_code_sha256"] == code, os.path.basename(path)
        ratio = float(kv["hbm_bytes_per_launch"]) / float(kv["algorithmic_bytes_per_launch"])
        assert ratio == pytest.approx(float(kv["traffic_over_algorithmic"]), abs=1e-6)
        assert 0.999 < ratio < 1.001, os.path.basename(path)
