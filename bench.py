"""Benchmark of the sharded update on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole hot path over one batch of synthetic input:
reduce-scatter of N=4 ranks' BF16 gradients into 4 FP32 owner shards (one
launch), the fused Adam/AdamW update of each owner shard (4 launches), and the
all-gather of the 4 BF16 working shards into the full view (one launch).  The
default workload is one 7B-class transformer layer (d=4096, ffn=11008,
202,375,168 parameters) with ranks weighted by token counts 4096/3072/4096/2048
and AdamW (wd=0.1).  Inputs are resident in HBM before the timed region.

Prints ONE JSON line: params updated per second (value), the step time, the
achieved algorithmic HBM bandwidth, the roofline entry of the dominant kernel
(the Adam update) measured with HIP events on the launch stream, and the CPU
oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X published peak HBM3E bandwidth
KERNEL_SRC = os.path.join(ROOT, "zero_sharded_optimizer_reduce_amd", "csrc", "kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "adam_shard_step_layer7b_traffic.txt")

# algorithmic HBM bytes per parameter (N = 4 ranks)
B_RS = lambda n: 2 * n + 4      # read N BF16 contributions, write one FP32 sum
B_ADAM = 30                     # read g, p, m, v (16 B); write p, m, v (12 B) + BF16 (2 B)
B_AG = 4                        # read and write one BF16 value


def _kernel_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def _traffic(launch_params: int):
    """HBM bytes per Adam launch from the committed rocprofv3 counter summary,
    or None if there is none or the kernel source changed since it was taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256") != _kernel_hash():
        return None
    try:
        if int(kv["params_per_launch"]) != launch_params:
            return None
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _cpu_baseline(target_s: float):
    """The oracle, as it stands, on 2^22-parameter slices of the same workload
    (reduce-scatter of 4 count-weighted BF16 ranks, AdamW, BF16 pack, gather),
    repeated until target_s seconds of CPU work.  numpy's element-wise ufuncs
    run on one thread."""
    import numpy as np

    import oracle
    import synthetic as S
    from synthetic.workloads import LAYER_7B as wl

    n, chunk = wl.n_ranks, 1 << 22
    grads = S.host_rank_grads(wl.seed, n, chunk, wl.grad_sigma, S.rank_scales(wl.seed, n))
    p, m, v = S.host_state(wl.seed + 1, chunk, wl.master_sigma)
    w = oracle.weights_from_counts(wl.extra["token_counts"])
    sc = oracle.adam_scalars(wl.lr, wl.beta1, wl.beta2, wl.eps, wl.weight_decay, 1)
    s = chunk // n
    done, reps = 0, 0
    t0 = time.perf_counter()
    while True:
        outs, view = oracle.sharded_step(grads, w, [p[k * s:(k + 1) * s] for k in range(n)],
                                         [m[k * s:(k + 1) * s] for k in range(n)],
                                         [v[k * s:(k + 1) * s] for k in range(n)], sc)
        done += chunk
        reps += 1
        el = time.perf_counter() - t0
        if el >= target_s:
            break
    del outs, view
    return {"value": done / el, "unit": "params/s", "cores": 1, "kind": "oracle",
            "sample": (f"oracle sharded step on a 2^22-param slice of the 7B-class layer "
                       f"(4 count-weighted BF16 ranks, AdamW, BF16 pack, all-gather), "
                       f"{reps} repetitions in {el:.1f} s on 1 thread (numpy ufuncs); "
                       f"host has {os.cpu_count()} CPUs")}


def run_layer7b(args):
    import numpy as np
    import torch

    import synthetic as S
    from synthetic.workloads import LAYER_7B as wl
    import zero_sharded_optimizer_reduce_amd as z
    from zero_sharded_optimizer_reduce_amd.drivers import ShardedStep

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    n = wl.n_ranks
    st = ShardedStep(S.unit_numels(S.workloads.layer_7b_tensors()), n, device=dev)
    gen = S.DeviceGen(wl.seed)
    st.load_master(gen.normal_(torch.empty(st.psi_pad, device=dev), wl.master_sigma, 0))
    scales = S.rank_scales(wl.seed, n)
    grads = [torch.empty(st.psi_pad, dtype=torch.bfloat16, device=dev) for _ in range(n)]
    tmp = torch.empty(st.psi_pad, dtype=torch.float32, device=dev)
    for r in range(n):
        gen.bf16_normal_(grads[r], wl.grad_sigma, 1, r, scale=scales[r], tmp=tmp)
    del tmp
    w = z.zero_rank_weights(wl.extra["token_counts"], n)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()

    t = 0
    for _ in range(args.warmup):
        t += 1
        st.step(grads, w, wl.hparams(step=t))
    torch.cuda.synchronize()

    E = lambda: torch.cuda.Event(enable_timing=True)
    ev = [[E() for _ in range(2 + 2 * n + 2)] for _ in range(args.steps)]
    start, stop = E(), E()
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        t += 1
        hp = wl.hparams(step=t)
        e = ev[i]
        e[0].record(stream)
        st.reduce_scatter(grads, w)
        e[1].record(stream)
        for k in range(n):
            e[2 + 2 * k].record(stream)
            z.zero_adam_shard_step(st.master[k], st.exp_avg[k], st.exp_avg_sq[k], st.bf16[k], st.grad[k], hp)
            e[3 + 2 * k].record(stream)
        e[2 + 2 * n].record(stream)
        st.all_gather()
        e[3 + 2 * n].record(stream)
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall0
    total_ms = start.elapsed_time(stop)
    ms_step = total_ms / args.steps
    rs_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    adam_ms = float(np.mean([e[2 + 2 * k].elapsed_time(e[3 + 2 * k]) for e in ev for k in range(n)]))
    ag_ms = float(np.mean([e[2 + 2 * n].elapsed_time(e[3 + 2 * n]) for e in ev]))

    psi, S_ = st.psi, st.shard
    step_bytes = (B_RS(n) + B_ADAM + B_AG) * st.psi_pad
    adam_bytes = B_ADAM * S_
    achieved = adam_bytes / (adam_ms * 1e-3) / 1e9
    traffic = _traffic(S_)
    out = {
        "metric": "params updated/sec per step and achieved HBM GB/s (% of MI355X peak), N=4",
        "value": psi / (ms_step * 1e-3),
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.description, "params": psi, "n_ranks": n,
                   "storage": "bf16 grads and working weights, fp32 master/m/v",
                   "step": "reduce-scatter + 4 owner Adam updates + all-gather"},
        "hbm_gbs_algorithmic": step_bytes / (ms_step * 1e-3) / 1e9,
        "hbm_frac_of_peak": step_bytes / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "wall_s_timed": wall,
        "kernels": {
            "reduce_scatter": {"ms": rs_ms, "bytes": B_RS(n) * st.psi_pad,
                               "gbs": B_RS(n) * st.psi_pad / (rs_ms * 1e-3) / 1e9},
            "adam_shard_step": {"ms": adam_ms, "bytes": adam_bytes, "gbs": achieved},
            "all_gather": {"ms": ag_ms, "bytes": B_AG * st.psi_pad,
                           "gbs": B_AG * st.psi_pad / (ag_ms * 1e-3) / 1e9},
        },
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS,
                     "traffic": traffic, "kernel": "adam_shard_step",
                     "algorithmic_bytes_per_launch": adam_bytes},
    }
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="layer7b_weighted_adamw")
    ap.add_argument("--cpu-baseline-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (--gpus {args.gpus} requested): the ranks are "
              "simulated as buffers in one GPU's HBM and no multi-GPU path is built.", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    from zero_sharded_optimizer_reduce_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    if args.workload != "layer7b_weighted_adamw":
        print(f"unknown workload {args.workload}", file=sys.stderr)
        sys.exit(2)
    out = run_layer7b(args)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = _cpu_baseline(args.cpu_baseline_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
