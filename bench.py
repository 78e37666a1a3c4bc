"""Benchmark of the sharded update on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole hot path over one batch of synthetic input.
The default workload is the largest one that fits one GPU: the ZeRO-3
per-unit chain of an 8B Llama-like model (34 units: embedding, 32 layers with
d=4096, ffn=14336, GQA kv_dim=1024, lm_head 128256x4096; 8,029,995,008
parameters) with N=4 simulated ranks.  Forward: every unit's 4 BF16 owner
shards are all-gathered into a temporary view, which is released.  Backward,
units in reverse order: reduce-scatter of the 4 ranks' BF16 contributions
into 4 FP32 owner shards, then the 4 owners' fused Adam updates (FP32 master,
m, v and the BF16 working shard).  Inputs are resident in HBM before the timed
region.  The same line carries, under extra keys, the figures of the
7B-class layer (d=4096, ffn=11008, 202,375,168 parameters, ranks weighted by
token counts, AdamW wd=0.1), of one owner's 2.0e9-parameter share in 64M
buckets and of the host-offloaded shard, each measured in a child process
that runs before this process touches the GPU (--chain-only leaves them out).

Other workloads (--workload): tiny_flat_1m, layer7b_weighted_adamw,
owner_share_8b_buckets (one owner's 2.0e9-parameter share in 64M buckets),
offload_owner_8b_two_slots (host-offloaded gradient shard through two device
slots), copy_calibration (copies of known size for the byte counters).

Prints ONE JSON line: params updated per second (value), the step time, the
achieved algorithmic HBM bandwidth, the roofline entry of the dominant kernel
measured with HIP events on the launch stream inside the timed region, and
the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import contextlib
import gc
import hashlib
import json
import os
import struct
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X published peak HBM3E bandwidth
LIBZERO = os.path.join(ROOT, "zero_sharded_optimizer_reduce_amd", "libzero.so")
PROFILES = os.path.join(ROOT, "profiles")
METRIC = "params updated/sec per step and achieved HBM GB/s (% of MI355X peak), N=4"

# algorithmic HBM bytes per parameter
B_RS = lambda n: 2 * n + 4      # read N BF16 contributions, write one FP32 sum
B_RS_ACC = lambda n: 2 * n + 8  # ... plus read the FP32 accumulator
B_ADAM = 30                     # read g, p, m, v (16 B); write p, m, v (12 B) + BF16 (2 B)
B_AG = 4                        # read and write one BF16 value


def _elf_section_bytes(d: bytes, name: str, what: str = "ELF") -> bytes:
    """The bytes of section `name` of a little-endian ELF64 image."""
    if d[:4] != b"\x7fELF" or d[4] != 2:
        raise ValueError(f"{what} is not an ELF64 image")
    shoff, = struct.unpack_from("<Q", d, 0x28)
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", d, 0x3A)

    def header(i):
        nm, _typ, _flags, _addr, off, size = struct.unpack_from("<IIQQQQ", d, shoff + i * shentsize)
        return nm, off, size

    strtab = header(shstrndx)[1]
    for i in range(shnum):
        nm, off, size = header(i)
        if d[strtab + nm: d.index(b"\0", strtab + nm)] == name.encode():
            return d[off:off + size]
    raise ValueError(f"{what} has no {name} section")


def _elf_section(path: str, name: str) -> bytes:
    with open(path, "rb") as f:
        return _elf_section_bytes(f.read(), name, path)


def device_code_hash() -> str:
    """sha256 of the machine code libzero.so carries for the GPU: for every
    amdgcn code object in its .hip_fatbin section (clang offload bundles), the
    .text section (the instructions) and the .rodata section (the kernel
    descriptors: resources, LDS, entry offsets).  Symbol and string tables
    are left out: they carry compilation-unit IDs derived from the source
    path, so the same sources built in another directory keep the hash, and
    so do edits that leave the machine code alone (comments, host code)."""
    fat = _elf_section(LIBZERO, ".hip_fatbin")
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    h = hashlib.sha256()
    objects = 0
    pos = fat.find(magic)
    while pos >= 0:
        count, = struct.unpack_from("<Q", fat, pos + len(magic))
        q = pos + len(magic) + 8
        for _ in range(count):
            off, size, tlen = struct.unpack_from("<QQQ", fat, q)
            triple = fat[q + 24:q + 24 + tlen]
            q += 24 + tlen
            if b"amdgcn" in triple:
                co = fat[pos + off:pos + off + size]
                h.update(triple)
                for sec in (".text", ".rodata"):
                    h.update(_elf_section_bytes(co, sec, triple.decode(errors="replace")))
                objects += 1
        pos = fat.find(magic, pos + len(magic))
    if objects == 0:
        raise ValueError(f"{LIBZERO} carries no amdgcn code object")
    return h.hexdigest()


def _traffic(kernel: str, workload: str, launch_params: int):
    """(HBM bytes per launch, source note) of `kernel` from the committed
    rocprofv3 counter summary, or (None, reason) if there is none, or the
    library's device code has changed since it was taken, or it covers
    another launch size."""
    name = f"{kernel}_{workload}_traffic.txt"
    path = os.path.join(PROFILES, name)
    if not os.path.exists(path):
        return None, f"no counter summary profiles/{name}"
    kv = {}
    for line in open(path):
        if ":" in line and not line.lstrip().startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    try:
        code = device_code_hash()
    except (OSError, ValueError) as e:
        return None, f"device code of libzero.so not readable ({e})"
    if kv.get("device_code_sha256") != code:
        return None, f"profiles/{name} was taken on other device code"
    try:
        if int(kv["params_per_launch"]) != launch_params:
            return None, f"profiles/{name} covers another launch size"
        return float(kv["hbm_bytes_per_launch"]), (
            f"profiles/{name}: FETCH_SIZE and WRITE_SIZE from two earlier rocprofv3 counter runs on "
            f"this device code (sha256 {code[:12]}), not from this run")
    except (KeyError, ValueError):
        return None, f"profiles/{name} is incomplete"


def _roofline(kernel, workload, ms, params, timing):
    achieved = B_ADAM * params / (ms * 1e-3) / 1e9
    traffic, source = _traffic(kernel, workload, params)
    return {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS, "traffic": traffic, "traffic_source": source,
            # the counters' bytes over the same measured launch time
            "traffic_gbs": None if traffic is None else traffic / (ms * 1e-3) / 1e9,
            "kernel": kernel, "params_per_launch": params, "algorithmic_bytes_per_launch": B_ADAM * params,
            "launch_ms": ms, "timing": timing}


@contextlib.contextmanager
def no_gc():
    """A timed region without Python's cyclic garbage collector: a full
    collection over the objects that torch, numpy and the CPU baseline leave
    (about 170k) pauses the launching thread for about 40 ms.  The host
    queues a step in well under a millisecond but is only a few tens of
    milliseconds ahead of the GPU early in a loop, so such a pause lets the
    GPU run dry (measured: one 40 ms collection at step 19 of the 7B-layer
    loop added 0.15 ms to the average step).  Garbage is collected before
    the region instead."""
    gc.collect()
    enabled = gc.isenabled()
    gc.disable()
    try:
        yield
    finally:
        if enabled:
            gc.enable()


def _mean(xs):
    return float(sum(xs) / max(1, len(xs)))


class Timer:
    """HIP events on the launch stream (the current torch stream, which every
    library call here is given)."""

    def __init__(self):
        import torch
        self.torch = torch
        self.stream = torch.cuda.current_stream()
        self.spans = {}

    def ev(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record(self.stream)
        return e

    def span(self, name, a, b):
        self.spans.setdefault(name, []).append((a, b))

    def ms(self, name):
        return _mean([a.elapsed_time(b) for a, b in self.spans.get(name, [])])


def event_overhead_ms(T, fn, reps=20, rounds=3):
    """GPU time that one event recorded between two kernels adds to the
    stream: reps back-to-back calls of fn timed with no event between them,
    then with an event after every call; the difference over reps, median of
    `rounds` alternations.  Spans taken between events inside a step carry
    one such gap each, which the breakdowns subtract."""
    torch = T.torch
    for _ in range(2):
        fn()
    torch.cuda.synchronize()
    est = []
    with no_gc():
        for _ in range(rounds):
            a = T.ev()
            for _ in range(reps):
                fn()
            b = T.ev()
            c = T.ev()
            for _ in range(reps):
                fn()
                d = T.ev()
            torch.cuda.synchronize()
            est.append((c.elapsed_time(d) - a.elapsed_time(b)) / reps)
    est.sort()
    return max(0.0, est[len(est) // 2])


def copy_ceiling_gbs(nbytes=1 << 30, reps=20):
    """Same-run ceiling: the library's copy kernel (all-gather of one shard)
    over nbytes, read + write bytes per second."""
    import torch

    import zero_sharded_optimizer_reduce_amd as z
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    for _ in range(3):
        z.zero_all_gather_layer([src], dst)
    T = Timer()
    with no_gc():
        a = T.ev()
        for _ in range(reps):
            z.zero_all_gather_layer([src], dst)
        b = T.ev()
        torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    del src, dst
    return 2 * nbytes / (ms * 1e-3) / 1e9


def _base(workload_desc, value, ms_step, args, extra_cfg=None):
    cfg = {"workload": workload_desc}
    cfg.update(extra_cfg or {})
    return {"metric": METRIC, "value": value, "unit": "params/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "f32", "data": "synthetic", "config": cfg}


# --------------------------------------------------------------------------- CPU baseline
CPU_SLICE = 1 << 22


def _cpu_slice_step(kind: str, slice_index: int):
    """One oracle step on one 2^22-parameter slice of a workload, its inputs
    drawn on the host as that workload draws them: returns a callable that
    runs the step (its results are discarded; the inputs stay as drawn)."""
    import numpy as np

    import oracle
    import synthetic as S
    from synthetic.workloads import CHAIN_8B, LAYER_7B, OFFLOAD_8B, OWNER_8B

    wl = {"layer7b_weighted_adamw": LAYER_7B, "zero3_chain_llama8b": CHAIN_8B,
          "owner_share_8b_buckets": OWNER_8B, "offload_owner_8b_two_slots": OFFLOAD_8B}[kind]
    n = wl.n_ranks
    seed = wl.seed + 1000 * slice_index
    p, m, v = S.host_state(seed + 1, CPU_SLICE, wl.master_sigma, wl.m_sigma, wl.v_sigma)
    sc = oracle.adam_scalars(wl.lr, wl.beta1, wl.beta2, wl.eps, wl.weight_decay, wl.step0)
    if kind == "owner_share_8b_buckets":
        # one owner's pre-sliced contributions: the reduce and the owner's update
        grads = S.host_rank_grads(seed, n, CPU_SLICE, wl.grad_sigma)
        w = oracle.weights_mean(n)
        return lambda: oracle.adam_step(p, m, v, oracle.reduce_full(grads, w), sc)
    if kind == "offload_owner_8b_two_slots":
        # M micro-batches accumulated, then the owner's update
        M = wl.extra["micro_batches"]
        per_mb = [S.host_rank_grads(seed + 7 * mb, n, CPU_SLICE, wl.grad_sigma) for mb in range(M)]
        w = np.full(n, 1.0 / (n * M), np.float32)
        return lambda: oracle.adam_step(p, m, v, oracle.offload_accumulate(per_mb, w), sc)
    if kind == "layer7b_weighted_adamw":
        grads = S.host_rank_grads(seed, n, CPU_SLICE, wl.grad_sigma, S.rank_scales(wl.seed, n))
        w = oracle.weights_from_counts(wl.extra["token_counts"])
    else:   # zero3_chain_llama8b: slices of the embedding unit and of layer 0 in turn
        seed += 0 if slice_index % 2 == 0 else 1
        grads = S.host_rank_grads(seed, n, CPU_SLICE, wl.grad_sigma)
        w = oracle.weights_mean(n)
    s = CPU_SLICE // n
    shards = [[x[k * s:(k + 1) * s] for k in range(n)] for x in (p, m, v)]
    return lambda: oracle.sharded_step(grads, w, *shards, sc)


def _cpu_slice_worker(kind: str, slice_index: int, target_s: float):
    """One process: the oracle's step on one 2^22-parameter slice of the
    workload (for the flat and chain workloads the sharded step: the
    reduce-scatter, the N owners' updates with the BF16 pack and the
    all-gather), repeated until target_s seconds have passed.  Returns
    (parameters stepped, seconds)."""
    step = _cpu_slice_step(kind, slice_index)
    done = 0
    t0 = time.perf_counter()
    while True:
        step()
        done += CPU_SLICE
        el = time.perf_counter() - t0
        if el >= target_s:
            return done, el


CPU_SAMPLES = {
    "layer7b_weighted_adamw": ("2^22-param slices of the 7B-class layer (4 count-weighted BF16 ranks, AdamW "
                               "wd=0.1; the sharded step: reduce-scatter, owner updates with the BF16 pack, "
                               "all-gather)", 202_375_168),
    "zero3_chain_llama8b": ("2^22-param slices cut alternately from the embedding unit and from layer 0 of the "
                            "8B chain (4 mean-weighted BF16 ranks, Adam t=1, wd=0; the sharded step: "
                            "reduce-scatter, owner updates with the BF16 pack, all-gather)", 8_029_995_008),
    "owner_share_8b_buckets": ("2^22-param slices of the owner's 2.0e9 share (4 mean-weighted BF16 "
                               "contributions, Adam t=1000 from a mid-run state, wd=0.1; the reduce and the "
                               "owner's update)", 2_000_000_000),
    "offload_owner_8b_two_slots": ("2^22-param slices of the offloaded 2.0e9 shard (4 micro-batches of 4 BF16 "
                                   "contributions at w=1/16 accumulated, then the owner's Adam t=1 update; the "
                                   "host link is not modelled)", 2_000_000_000),
}


def cpu_baseline(kind: str, target_s: float):
    """The oracle, as it stands, on 2^22-parameter slices of the workload: first
    in this process on one thread for target_s seconds, then in one process
    per available core (at most 16), each on its own slice, for target_s
    seconds.  The slices are independent, as the shards are, and every step
    of the path is element-wise, so the time of a whole step is the
    parameter count over the measured rate: the extrapolation is stated in
    the result.  Runs before the GPU is touched."""
    import concurrent.futures as cf
    import multiprocessing as mp
    import platform

    what, psi = CPU_SAMPLES[kind]
    done1, el1 = _cpu_slice_worker(kind, 0, target_s)
    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    with cf.ProcessPoolExecutor(cores, mp_context=mp.get_context("spawn")) as ex:
        # one warm-up task per worker so that interpreter and import time stay out
        list(ex.map(_cpu_slice_worker, [kind] * cores, range(cores), [0.0] * cores))
        res = list(ex.map(_cpu_slice_worker, [kind] * cores, range(cores), [target_s] * cores))
    done_all = sum(r[0] for r in res)
    wall = max(r[1] for r in res)      # the workers' step loops run concurrently
    model = platform.processor() or platform.machine()
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    rate, rate1 = done_all / wall, done1 / el1
    return {"value": rate, "unit": "params/s", "cores": cores, "kind": "oracle",
            "sample": (f"the oracle's step on {what}: {cores} processes, one slice each, "
                       f"{done_all // CPU_SLICE} slice-steps, the "
                       f"slowest process's loop {wall:.1f} s; numpy ufuncs, one thread per process; {model}, "
                       f"{os.cpu_count()} CPUs visible, {cores} in the affinity mask used (capped at 16). "
                       f"Extrapolated by parameter count: one {psi:,}-parameter step would take "
                       f"{psi / rate:.1f} s on {cores} cores and {psi / rate1:.1f} s on one."),
            "extrapolated_step_s": psi / rate,
            "single_thread": {"value": rate1, "unit": "params/s", "cores": 1,
                              "sample": f"{done1 // CPU_SLICE} slice-steps in {el1:.1f} s on one thread",
                              "extrapolated_step_s": psi / rate1}}


# --------------------------------------------------------------------------- flat units
SAMPLE_EVERY = 4   # steps between the sampled per-kernel event pairs


def run_flat(args, wl, numels, grad_scales=None, counts=None):
    """Timed region: args.steps steps bracketed by two events, with events
    between the reduce-scatter, the 4 owner updates and the all-gather on
    every SAMPLE_EVERY-th step only, so that the step time carries few
    events; the breakdown subtracts the GPU time of one event between two
    kernels, measured in the same run."""
    import torch

    import synthetic as S
    import zero_sharded_optimizer_reduce_amd as z
    from zero_sharded_optimizer_reduce_amd.drivers import ShardedStep

    dev = torch.device("cuda:0")
    n = wl.n_ranks
    st = ShardedStep(numels, n, device=dev)
    gen = S.DeviceGen(wl.seed)
    st.load_master(gen.normal_(torch.empty(st.psi_pad, device=dev), wl.master_sigma, 0))
    scales = grad_scales or [1.0] * n
    grads = [torch.empty(st.psi_pad, dtype=torch.bfloat16, device=dev) for _ in range(n)]
    tmp = torch.empty(st.psi_pad, dtype=torch.float32, device=dev)
    for r in range(n):
        gen.bf16_normal_(grads[r], wl.grad_sigma, 1, r, scale=scales[r], tmp=tmp)
    del tmp
    w = z.zero_rank_weights(counts, n)
    T = Timer()
    t = 0

    def timed(step_fn, phase_name):
        nonlocal t
        for _ in range(args.warmup):
            t += 1
            step_fn(wl.hparams(step=t), None)
        torch.cuda.synchronize()
        with no_gc():
            t0 = time.perf_counter()
            start = T.ev()
            for i in range(args.steps):
                t += 1
                step_fn(wl.hparams(step=t), phase_name if i % SAMPLE_EVERY == 0 else None)
            stop = T.ev()
            torch.cuda.synchronize()
            wall = time.perf_counter() - t0
        return start.elapsed_time(stop) / args.steps, wall

    def sep_step(hp, sample):
        if not sample:
            st.reduce_scatter(grads, w)
            st.update(hp)
            st.all_gather()
            return
        a = T.ev()
        st.reduce_scatter(grads, w)
        b = T.ev()
        st.update(hp)
        c = T.ev()
        st.all_gather()
        T.span("rs", a, b)
        T.span(sample, b, c)
        T.span("ag", c, T.ev())

    def fused_step(hp, sample):
        a = T.ev() if sample else None
        z.zero_reduce_scatter_adam(grads, w, st.master, st.exp_avg, st.exp_avg_sq, st.bf16, hp)
        if sample:
            T.span(sample, a, T.ev())
        st.all_gather()

    ms_step, wall = timed(sep_step, "update4")
    adam_ms = T.ms("update4") / n
    ev_ms = event_overhead_ms(T, st.all_gather)
    rs_ms, ag_ms = T.ms("rs") - ev_ms, T.ms("ag") - ev_ms
    adam_corr = (T.ms("update4") - ev_ms) / n
    pad = st.psi_pad
    step_bytes = (B_RS(n) + B_ADAM + B_AG) * pad
    out = _base(wl.description, st.psi / (ms_step * 1e-3), ms_step, args,
                {"params": st.psi, "n_ranks": n, "storage": "bf16 grads and working weights, fp32 master/m/v",
                 "step": "reduce-scatter + 4 owner Adam updates + all-gather"})
    out.update({
        "hbm_gbs_algorithmic": step_bytes / (ms_step * 1e-3) / 1e9,
        "hbm_frac_of_peak": step_bytes / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "wall_s_timed": wall,
        "kernels": {
            "timing": (f"events between the step's kernel groups on every {SAMPLE_EVERY}th step of the timed "
                       "region, each span less the measured GPU time of one event between two kernels"),
            "event_overhead_ms": ev_ms,
            "reduce_scatter": {"ms": rs_ms, "bytes": B_RS(n) * pad, "gbs": B_RS(n) * pad / (rs_ms * 1e-3) / 1e9,
                               "launches": n},
            "adam_shard_step": {"ms": adam_corr, "bytes": B_ADAM * st.shard,
                                "gbs": B_ADAM * st.shard / (adam_corr * 1e-3) / 1e9, "per": "owner launch"},
            "all_gather": {"ms": ag_ms, "bytes": B_AG * pad, "gbs": B_AG * pad / (ag_ms * 1e-3) / 1e9},
            "sum_ms": rs_ms + n * adam_corr + ag_ms,
        },
        "roofline": _roofline("adam_shard_step", wl.name, adam_ms, st.shard,
                              f"HIP events on the launch stream around the 4 owner updates on every "
                              f"{SAMPLE_EVERY}th step of the timed region, divided by 4"),
    })
    # the same step with the fused reduce-scatter + update kernel (reduced
    # gradient kept in registers) and the all-gather
    f_ms, _ = timed(fused_step, "fused4")
    fk = T.ms("fused4")
    out["fused_variant"] = {
        "ms_per_step": f_ms, "value": st.psi / (f_ms * 1e-3),
        "step": "fused reduce-scatter + owner updates (one launch per owner) + all-gather, 38 B/param",
        "fused_kernel": {"ms": fk / n, "bytes": (2 * n + 26) * st.shard,
                         "gbs": (2 * n + 26) * pad / (fk * 1e-3) / 1e9},
        "hbm_gbs_algorithmic": (2 * n + 26 + B_AG) * pad / (f_ms * 1e-3) / 1e9,
    }

    # the same fused step, also storing the reduced FP32 shards: every output of
    # the separate-kernel step, 42 B/param
    def fused_gout_step(hp, sample):
        a = T.ev() if sample else None
        z.zero_reduce_scatter_adam(grads, w, st.master, st.exp_avg, st.exp_avg_sq, st.bf16, hp, grad_out=st.grad)
        if sample:
            T.span(sample, a, T.ev())
        st.all_gather()

    fg_ms, _ = timed(fused_gout_step, "fused4g")
    fgk = T.ms("fused4g")
    out["fused_variant_storing_grad"] = {
        "ms_per_step": fg_ms, "value": st.psi / (fg_ms * 1e-3),
        "step": "fused reduce-scatter + owner updates that also store the reduced FP32 shards + all-gather, "
                "42 B/param (the same outputs as the separate kernels)",
        "fused_kernel": {"ms": fgk / n, "bytes": (2 * n + 30) * st.shard,
                         "gbs": (2 * n + 30) * pad / (fgk * 1e-3) / 1e9},
        "hbm_gbs_algorithmic": (2 * n + 30 + B_AG) * pad / (fg_ms * 1e-3) / 1e9,
    }
    # the separate-kernel step captured once into a HIP graph and replayed
    # (the graph's first kernel takes the step's scalars from a pinned ring)
    from zero_sharded_optimizer_reduce_amd.drivers import GraphedStep
    gs = GraphedStep(st, grads, w)
    gr_ms, _ = timed(lambda hp, sample: gs.step(hp), None)
    out["graph_variant"] = {
        "ms_per_step": gr_ms, "value": st.psi / (gr_ms * 1e-3),
        "step": "scalar fetch from a pinned ring + reduce-scatter + 4 owner updates (scalars read from "
                "device memory) + all-gather, captured once and replayed",
        "hbm_gbs_algorithmic": step_bytes / (gr_ms * 1e-3) / 1e9}
    del gs
    out["next_rows"] = _next_rows(args, st, grads, w, wl, timed, T)
    out["copy_ceiling_gbs_same_run"] = copy_ceiling_gbs()
    return out


def _next_rows(args, st, grads, w, wl, timed, T):
    """The optional rows beyond the sharded step, each timed on the same
    buffers: the step with a global gradient-norm clip, the reduce with FP32
    contributions, and the reduce in accumulate mode."""
    import torch

    import zero_sharded_optimizer_reduce_amd as z
    from zero_sharded_optimizer_reduce_amd import _lib

    n, pad = st.n, st.psi_pad
    ws = torch.empty(n * _lib.ZERO_NORM_BLOCKS, dtype=torch.float64, device="cuda")
    norm_sq = torch.empty(1, dtype=torch.float64, device="cuda")
    coef = torch.empty(1, dtype=torch.float32, device="cuda")

    def clipped_step(hp, sample):
        st.reduce_scatter(grads, w)
        a = T.ev() if sample else None
        z.zero_grad_norm_sq(st.grad, ws, norm_sq, max_norm=1.0, clip_coef_out=coef)
        if sample:
            T.span("norm", a, T.ev())
        for k in range(n):
            z.zero_adam_shard_step_scaled(st.master[k], st.exp_avg[k], st.exp_avg_sq[k], st.bf16[k], st.grad[k],
                                          coef, hp)
        st.all_gather()

    c_ms, _ = timed(clipped_step, "norm")
    norm_ms = T.ms("norm")
    res = {"grad_norm_clip": {
        "ms_per_step": c_ms, "value": st.psi / (c_ms * 1e-3),
        "step": "reduce-scatter + global gradient norm (FP64, fixed order) and clip coefficient (max_norm 1.0) "
                "+ 4 owner updates on the scaled gradient + all-gather, 50 B/param",
        "hbm_gbs_algorithmic": 50 * pad / (c_ms * 1e-3) / 1e9,
        "norm_kernels": {"ms": norm_ms, "bytes": 4 * pad, "gbs": 4 * pad / (norm_ms * 1e-3) / 1e9,
                         "timing": f"event pair around the norm call on every {SAMPLE_EVERY}th timed step"}}}

    def run_calls(fn, reps):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        with no_gc():
            a = T.ev()
            for _ in range(reps):
                fn()
            b = T.ev()
            torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    reps = max(4, args.steps // 4)
    acc_ms = run_calls(lambda: z.zero_reduce_scatter(grads, w, st.grad, accumulate=True), reps)
    res["reduce_scatter_accumulate"] = {
        "ms": acc_ms, "bytes": B_RS_ACC(n) * pad, "gbs": B_RS_ACC(n) * pad / (acc_ms * 1e-3) / 1e9,
        "what": "shard += reduction of the 4 BF16 contributions (micro-batch accumulation), 4 owner launches"}
    g32 = [g.float() for g in grads]
    f_ms = run_calls(lambda: z.zero_reduce_scatter_f32(g32, w, st.grad), reps)
    res["reduce_scatter_f32"] = {
        "ms": f_ms, "bytes": (4 * n + 4) * pad, "gbs": (4 * n + 4) * pad / (f_ms * 1e-3) / 1e9,
        "what": "reduce-scatter of 4 FP32 contributions (gradients kept in FP32), 4 owner launches"}
    del g32, ws
    torch.cuda.empty_cache()
    return res


def run_layer7b(args):
    import synthetic as S
    from synthetic.workloads import LAYER_7B as wl
    return run_flat(args, wl, S.unit_numels(S.workloads.layer_7b_tensors()),
                    grad_scales=S.rank_scales(wl.seed, wl.n_ranks), counts=wl.extra["token_counts"])


def run_tiny(args):
    from synthetic.workloads import TINY as wl
    return run_flat(args, wl, [wl.psi])


# --------------------------------------------------------------------------- owner share, buckets
def run_owner_share(args):
    import torch

    import synthetic as S
    from synthetic import fill
    from synthetic.workloads import OWNER_8B as wl
    import zero_sharded_optimizer_reduce_amd as z
    from zero_sharded_optimizer_reduce_amd.drivers import BucketedOwnerStep

    n = wl.n_ranks
    st = BucketedOwnerStep(wl.psi, n, wl.extra["bucket"], device="cuda")
    gen = S.DeviceGen(wl.seed)
    tmp = torch.empty(wl.extra["bucket"], dtype=torch.float32, device="cuda")
    fill.fill_owner_share(gen, wl, st.master, st.exp_avg, st.exp_avg_sq, st.contrib, tmp)
    del tmp
    w = z.zero_rank_weights(None, n)
    T = Timer()
    B = st.bucket
    t = wl.step0 - 1

    def sep_step(hp, sample):
        for b, (lo, hi) in enumerate(st.bounds):
            g = st.grad_bucket[: hi - lo]
            if sample and b == 0:
                a = T.ev()
            z.zero_reduce_scatter([c[lo:hi] for c in st.contrib], w, [g])
            if sample and b == 0:
                m = T.ev()
            z.zero_adam_shard_step(st.master[lo:hi], st.exp_avg[lo:hi], st.exp_avg_sq[lo:hi], st.bf16[lo:hi], g, hp)
            if sample and b == 0:
                T.span("rs", a, m)
                T.span("adam", m, T.ev())

    def fused_step(hp, sample):
        for b, (lo, hi) in enumerate(st.bounds):
            if sample and b == 0:
                a = T.ev()
            z.zero_reduce_scatter_adam([c[lo:hi] for c in st.contrib], w, [st.master[lo:hi]], [st.exp_avg[lo:hi]],
                                       [st.exp_avg_sq[lo:hi]], [st.bf16[lo:hi]], hp)
            if sample and b == 0:
                T.span("fused", a, T.ev())

    def timed(step_fn):
        nonlocal t
        for _ in range(args.warmup):
            t += 1
            step_fn(wl.hparams(step=t), False)
        torch.cuda.synchronize()
        with no_gc():
            t0 = time.perf_counter()
            start = T.ev()
            for i in range(args.steps):
                t += 1
                step_fn(wl.hparams(step=t), i % SAMPLE_EVERY == 0)
            stop = T.ev()
            torch.cuda.synchronize()
            wall = time.perf_counter() - t0
        return start.elapsed_time(stop) / args.steps, wall

    assert st.bounds[0][1] - st.bounds[0][0] == B
    ms_step, wall = timed(sep_step)
    step_bytes = (B_RS(n) + B_ADAM) * wl.psi
    rs_ms, adam_ms = T.ms("rs"), T.ms("adam")
    out = _base(wl.description, wl.psi / (ms_step * 1e-3), ms_step, args,
                {"params": wl.psi, "n_ranks": n, "bucket": B, "buckets": len(st.bounds),
                 "step": "per bucket: reduce 4 pre-sliced contributions + owner Adam update"})
    out.update({
        "hbm_gbs_algorithmic": step_bytes / (ms_step * 1e-3) / 1e9,
        "hbm_frac_of_peak": step_bytes / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "wall_s_timed": wall,
        "kernels": {"reduce_scatter": {"ms": rs_ms, "bytes": B_RS(n) * B, "gbs": B_RS(n) * B / (rs_ms * 1e-3) / 1e9},
                    "adam_shard_step": {"ms": adam_ms, "bytes": B_ADAM * B, "gbs": B_ADAM * B / (adam_ms * 1e-3) / 1e9},
                    "timing": f"event pairs around the first bucket on every {SAMPLE_EVERY}th timed step"},
        "roofline": _roofline("adam_shard_step", wl.name, adam_ms, B,
                              f"HIP events on the launch stream around the first bucket's update on every "
                              f"{SAMPLE_EVERY}th step of the timed region"),
    })
    # the same step with the fused reduce + update kernel per bucket (34 B/param)
    f_ms, _ = timed(fused_step)
    fk = T.ms("fused")
    out["fused_variant"] = {"ms_per_step": f_ms, "value": wl.psi / (f_ms * 1e-3),
                            "hbm_gbs_algorithmic": (2 * n + 26) * wl.psi / (f_ms * 1e-3) / 1e9,
                            "fused_kernel": {"ms": fk, "bytes": (2 * n + 26) * B,
                                             "gbs": (2 * n + 26) * B / (fk * 1e-3) / 1e9}}
    out["copy_ceiling_gbs_same_run"] = copy_ceiling_gbs()
    return out


# --------------------------------------------------------------------------- ZeRO-3 chain
def _fused_kernel_entry(T, n, shard, regather):
    """The fused kernel on a layer unit: mean launch time over the sampled
    spans around every layer unit's 4 owner launches (the gather that
    regather adds is inside the span, so then only the span is given)."""
    ms = T.ms("layer_fused4")
    if regather or ms <= 0:
        return {"span_ms": ms}
    launch = ms / n
    b = (2 * n + 26) * shard
    return {"ms": launch, "bytes": b, "gbs": b / (launch * 1e-3) / 1e9,
            "frac_of_peak": b / (launch * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "timing": f"HIP events around every layer unit's 4 fused launches on every {SAMPLE_EVERY}th step, "
                      "mean over the 32 layers, divided by 4"}


CHAIN_SAMPLE_UNIT = 17   # layer 16 (unit 0 is the embedding, unit 33 the lm_head)


def run_chain(args):
    """One step: forward, for every unit in order, all-gather of the 4 BF16
    owner shards into a temporary view that is then released; backward, for
    every unit in reverse order, reduce-scatter of the 4 ranks' BF16
    contributions and the 4 owners' Adam updates.  The contributions (the
    output of a backward computation that is not part of the path) are drawn
    once, for the largest unit, before the timed region."""
    import torch

    import synthetic as S
    from synthetic import fill
    from synthetic.workloads import CHAIN_8B as wl
    import zero_sharded_optimizer_reduce_amd as z
    from zero_sharded_optimizer_reduce_amd.drivers import Zero3Chain

    n = wl.n_ranks
    torch.cuda.reset_peak_memory_stats()
    ch = Zero3Chain(wl.extra["units"], n, device="cuda")
    gen = S.DeviceGen(wl.seed)
    for k in range(n):
        fill.fill_normal_pieces(gen, ch.master[k], wl.master_sigma, fill.K_MASTER + 100 * k)
        for lo, hi in fill.pieces(ch.owner_numel):
            ch.bf16[k][lo:hi].copy_(ch.master[k][lo:hi])
    tmp = torch.empty(ch.max_pad, dtype=torch.float32, device="cuda")
    w = z.zero_rank_weights(None, n)
    T = Timer()
    U = len(ch.units)
    rg = bool(args.regather_bwd)
    fill.chain_unit_grads(gen, wl, 0, ch.grads, ch.max_pad, tmp)
    del tmp
    SU = CHAIN_SAMPLE_UNIT

    # sampled steps carry events around every layer unit's 4 owner updates
    # (the roofline kernel, averaged over all 32 layers as a kernel trace
    # averages it) and around the reduce and the gather of layer 16 and of
    # the embedding (the lm_head has the embedding's size)
    SAMPLED = {SU: "layer", 0: "embedding"}

    def step(t, sample=False, mid=None, fused=False):
        hp = wl.hparams(step=t)
        for u in range(U):                      # forward: gather, use, release
            if sample and u in SAMPLED:
                a = T.ev()
                ch.forward_unit(u)
                T.span(SAMPLED[u] + "_ag", a, T.ev())
            else:
                ch.forward_unit(u)
        if mid is not None:
            mid.append(T.ev())
        for u in reversed(range(U)):            # backward
            if fused:
                if sample and 1 <= u <= U - 2:
                    a = T.ev()
                    ch.backward_unit_fused(u, w, hp, regather=rg)
                    T.span("layer_fused4", a, T.ev())
                else:
                    ch.backward_unit_fused(u, w, hp, regather=rg)
                continue
            if rg:
                ch.forward_unit(u)
            is_layer = 1 <= u <= U - 2
            if sample and (u in SAMPLED or is_layer):
                a = T.ev() if u in SAMPLED else None
                ch.reduce_unit(u, w)
                b = T.ev()
                ch.update_unit(u, hp)
                c = T.ev()
                if a is not None:
                    T.span(SAMPLED[u] + "_rs", a, b)
                T.span("layer_update4" if is_layer else SAMPLED[u] + "_update4", b, c)
            else:
                ch.reduce_unit(u, w)
                ch.update_unit(u, hp)

    t = 0

    def timed(fused):
        nonlocal t
        for _ in range(args.warmup):
            t += 1
            step(t, fused=fused)
        torch.cuda.synchronize()
        with no_gc():
            t0 = time.perf_counter()
            marks = [T.ev()]
            for i in range(args.steps):
                t += 1
                step(t, sample=(i % SAMPLE_EVERY == 0), mid=marks, fused=fused)
                marks.append(T.ev())
            torch.cuda.synchronize()
            wall = time.perf_counter() - t0
        fwd = sum(marks[2 * i].elapsed_time(marks[2 * i + 1]) for i in range(args.steps)) / args.steps
        tot = marks[0].elapsed_time(marks[-1]) / args.steps
        return tot, fwd, wall

    ms_step, fwd_ms, wall = timed(False)
    bwd_ms = ms_step - fwd_ms
    adam_ms = T.ms("layer_update4") / n
    f_ms, _, _ = timed(True)
    psi_pad = sum(u[2] for u in ch.units)
    step_bytes = (B_RS(n) + B_ADAM + B_AG * (2 if rg else 1)) * psi_pad

    # per-kernel breakdown from the sampled steps' spans, each less the GPU
    # time of one event between two kernels (measured here)
    ev_ms = event_overhead_ms(T, lambda: ch.forward_unit(SU))
    kern = {"timing": (f"events on every {SAMPLE_EVERY}th step of the timed region: around every layer unit's "
                       "4 owner updates (the layer update is their mean over the 32 layers) and around the "
                       "reduce and the gather of layer 16 and of the embedding; each span less the measured GPU "
                       "time of one event between two kernels; the lm_head is counted with the embedding's "
                       "figures"),
            "event_overhead_ms": ev_ms}
    for name, u, count in (("layer", SU, U - 2), ("embedding", 0, 2)):
        pad, s = ch.units[u][2], ch.units[u][3]
        rs = T.ms(name + "_rs") - ev_ms
        ad = (T.ms("layer_update4" if name == "layer" else name + "_update4") - ev_ms) / n
        ag = T.ms(name + "_ag") - ev_ms
        kern[name] = {
            "units_per_step": count, "params_padded": pad, "shard": s,
            "reduce_scatter": {"ms": rs, "bytes": B_RS(n) * pad, "gbs": B_RS(n) * pad / (rs * 1e-3) / 1e9,
                               "launches": n},
            "adam_shard_step": {"ms": ad, "bytes": B_ADAM * s, "gbs": B_ADAM * s / (ad * 1e-3) / 1e9,
                                "per": "owner launch"},
            "all_gather": {"ms": ag, "bytes": B_AG * pad, "gbs": B_AG * pad / (ag * 1e-3) / 1e9}}
    kern["sum_ms"] = sum(k["units_per_step"] * (k["reduce_scatter"]["ms"] + n * k["adam_shard_step"]["ms"]
                                                + k["all_gather"]["ms"] * (2 if rg else 1))
                         for k in (kern["layer"], kern["embedding"]))
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated()
    persistent = sum(x.numel() * x.element_size() for x in ch.master + ch.exp_avg + ch.exp_avg_sq + ch.bf16)
    s_lay = ch.units[SU][3]
    out = _base(wl.description, wl.psi / (ms_step * 1e-3), ms_step, args,
                {"params": wl.psi, "n_ranks": n, "units": U, "regather_bwd": rg,
                 "step": "forward: 34 all-gathers into a released view; backward (reverse): "
                         + ("all-gather again, " if rg else "")
                         + "reduce-scatter + 4 owner Adam updates per unit; contributions generated "
                           "before the timed region"})
    out.update({
        "hbm_gbs_algorithmic": step_bytes / (ms_step * 1e-3) / 1e9,
        "hbm_frac_of_peak": step_bytes / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "algorithmic_bytes_per_step": step_bytes,
        "forward_ms": fwd_ms, "backward_ms": bwd_ms, "wall_s_timed": wall,
        "memory": {"persistent_bytes_all_owners": persistent,
                   "ledger_zero3_bytes_all_owners": 16 * wl.psi,
                   "peak_allocated_bytes": peak},
        "kernels": kern,
        "roofline": _roofline("adam_shard_step", wl.name, adam_ms, s_lay,
                              f"HIP events on the launch stream around the 4 owner updates of every layer unit "
                              f"on every {SAMPLE_EVERY}th step of the timed region: the mean span over the 32 "
                              "layers, divided by 4 (the span's one event gap is not subtracted here; "
                              "kernels.layer has the corrected figure)"),
        "fused_variant": {"ms_per_step": f_ms, "value": wl.psi / (f_ms * 1e-3),
                          "step": "backward per unit: fused reduce-scatter + owner update (one launch per "
                                  "owner, the reduced shards kept in registers)",
                          "hbm_gbs_algorithmic": (2 * n + 26 + B_AG * (2 if rg else 1)) * psi_pad
                          / (f_ms * 1e-3) / 1e9,
                          "fused_kernel_layer": _fused_kernel_entry(T, n, s_lay, rg)},
    })
    del ch
    gc.collect()
    torch.cuda.empty_cache()
    out["copy_ceiling_gbs_same_run"] = copy_ceiling_gbs()
    return out


# --------------------------------------------------------------------------- offload
def _pinned_copy_rates(nbytes):
    """Pinned host <-> device hipMemcpyAsync rates in this process: H2D alone,
    D2H alone, and both at once on two streams (GB/s)."""
    import torch
    h = torch.empty(nbytes // 4, dtype=torch.float32, pin_memory=True)
    h2 = torch.empty(nbytes // 4, dtype=torch.float32, pin_memory=True)
    d = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    d2 = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    res = {}
    for _ in range(2):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        with torch.cuda.stream(s1):
            d.copy_(h, non_blocking=True)
        torch.cuda.synchronize()
        res["h2d_gbs"] = nbytes / (time.perf_counter() - t0) / 1e9
        t0 = time.perf_counter()
        with torch.cuda.stream(s1):
            h.copy_(d, non_blocking=True)
        torch.cuda.synchronize()
        res["d2h_gbs"] = nbytes / (time.perf_counter() - t0) / 1e9
        t0 = time.perf_counter()
        with torch.cuda.stream(s1):
            d.copy_(h, non_blocking=True)
        with torch.cuda.stream(s2):
            h2.copy_(d2, non_blocking=True)
        torch.cuda.synchronize()
        res["bidir_gbs"] = 2 * nbytes / (time.perf_counter() - t0) / 1e9
    return res


def _shard_copy_rates(host, nbytes):
    """Pinned-copy rates on the offload shard's own pages: host-to-device
    from the shard's first nbytes, device-to-host into the next nbytes, each
    alone and both at once on two streams (GB/s).  The shard's contents are
    overwritten (the step rewrites every chunk at its first micro-batch)."""
    import torch
    words = nbytes // 4
    assert host.numel() >= 2 * words
    src_h, dst_h = host[:words], host[words:2 * words]
    d1 = torch.empty(words, dtype=torch.float32, device="cuda")
    d2 = torch.empty(words, dtype=torch.float32, device="cuda")
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    res = {}
    for _ in range(2):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        with torch.cuda.stream(s1):
            d1.copy_(src_h, non_blocking=True)
        torch.cuda.synchronize()
        res["h2d_gbs"] = nbytes / (time.perf_counter() - t0) / 1e9
        t0 = time.perf_counter()
        with torch.cuda.stream(s2):
            dst_h.copy_(d2, non_blocking=True)
        torch.cuda.synchronize()
        res["d2h_gbs"] = nbytes / (time.perf_counter() - t0) / 1e9
        t0 = time.perf_counter()
        with torch.cuda.stream(s1):
            d1.copy_(src_h, non_blocking=True)
        with torch.cuda.stream(s2):
            dst_h.copy_(d2, non_blocking=True)
        torch.cuda.synchronize()
        res["bidir_gbs"] = 2 * nbytes / (time.perf_counter() - t0) / 1e9
    del d1, d2
    return res


def _numa_placement(host):
    """NUMA nodes of the GPU, of this process's CPUs and of the pinned shard's
    pages (Linux sysfs, /proc/self/maps and /proc/self/numa_maps); None where
    the system does not say."""
    import glob

    import torch
    out = {"gpu_numa_node": None, "cpu_nodes": None, "shard_pages_by_node": None}
    try:
        p = torch.cuda.get_device_properties(0)
        bdf = f"{p.pci_domain_id:04x}:{p.pci_bus_id:02x}:{p.pci_device_id:02x}.0"
        out["gpu_pci"] = bdf
        out["gpu_numa_node"] = int(open(f"/sys/bus/pci/devices/{bdf}/numa_node").read().strip())
    except Exception as e:          # noqa: BLE001  (diagnostic only)
        out["gpu_numa_error"] = repr(e)[:120]
    try:
        nodes = {}
        for c in sorted(os.sched_getaffinity(0)):
            for d in glob.glob(f"/sys/devices/system/cpu/cpu{c}/node*"):
                k = int(d.rsplit("node", 1)[1])
                nodes[k] = nodes.get(k, 0) + 1
        out["cpu_nodes"] = nodes
    except Exception as e:          # noqa: BLE001
        out["cpu_nodes_error"] = repr(e)[:120]
    try:
        addr = host.data_ptr()
        start = None
        for line in open("/proc/self/maps"):
            lo, hi = (int(x, 16) for x in line.split()[0].split("-"))
            if lo <= addr < hi:
                start = lo
                out["shard_mapping"] = line.strip()[:160]
                break
        if start is not None:
            for line in open("/proc/self/numa_maps"):
                f = line.split()
                if int(f[0], 16) == start:
                    out["shard_numa_maps"] = line.strip()[:200]
                    pages = {int(x[1:].split("=")[0]): int(x.split("=")[1]) for x in f[2:]
                             if x.startswith("N") and "=" in x}
                    out["shard_pages_by_node"] = pages or None
                    break
    except Exception as e:          # noqa: BLE001
        out["shard_pages_error"] = repr(e)[:120]
    return out


def run_offload(args):
    import torch

    import synthetic as S
    from synthetic import fill
    from synthetic.workloads import OFFLOAD_8B as wl
    import zero_sharded_optimizer_reduce_amd as z
    from zero_sharded_optimizer_reduce_amd.drivers import OffloadStep

    n, M, C = wl.n_ranks, wl.extra["micro_batches"], wl.extra["chunk"]
    st = OffloadStep(wl.psi, n, C, device="cuda")
    gen = S.DeviceGen(wl.seed)
    tmp = torch.empty(C, dtype=torch.float32, device="cuda")
    fill.fill_normal_pieces(gen, st.master, wl.master_sigma, fill.K_MASTER)
    # producer: copies one of P pre-drawn contribution sets into the slot, as a
    # backward pass would write its gradient chunk
    P = 4
    pool = [torch.empty(n * C, dtype=torch.bfloat16, device="cuda") for _ in range(P)]
    for i, pbuf in enumerate(pool):
        fill.offload_contrib(gen, wl, 100 + i, 0, [pbuf[r * C:(r + 1) * C] for r in range(n)], tmp)
    del tmp
    w = [1.0 / (n * M)] * n

    def produce(mb, c, views):
        src = pool[(mb * 7 + c) % P]
        for r, vw in enumerate(views):
            vw.copy_(src[r * C: r * C + vw.numel()])

    step_ms = {}

    def timed(fuse_last):
        nonlocal t
        warm = []
        for _ in range(args.warmup):
            t += 1
            t0 = time.perf_counter()
            st.step(produce, M, w, wl.hparams(step=t), fuse_last=fuse_last)
            st.sync()
            warm.append(time.perf_counter() - t0)
        torch.cuda.synchronize()
        times = []
        with no_gc():
            for _ in range(args.steps):
                t += 1
                t0 = time.perf_counter()
                st.step(produce, M, w, wl.hparams(step=t), fuse_last=fuse_last)
                st.sync()
                torch.cuda.synchronize()
                times.append(time.perf_counter() - t0)
        step_ms["fused_last" if fuse_last else "literal"] = {"warmup": [1e3 * x for x in warm],
                                                             "timed": [1e3 * x for x in times]}
        return 1e3 * _mean(times)

    torch.cuda.synchronize()
    placement = _numa_placement(st.host)
    shard_before = _shard_copy_rates(st.host, 1 << 30)
    t = 0
    ms_step = timed(False)
    ms_fused = timed(True)
    shard_after = _shard_copy_rates(st.host, 1 << 30)
    link_bytes = 4 * wl.psi * (M + (M - 1) + 1)     # D2H every mb, H2D from mb 2, H2D stream-back
    link_fused = 4 * wl.psi * ((M - 1) + (M - 1))   # the last micro-batch never crosses the link
    fresh_after = _pinned_copy_rates(1 << 30)
    # The schedule at the measured pinned-copy rates: micro-batch 1 only copies
    # to the host, micro-batches 2..M copy both ways, the stream-back only
    # copies to the device.  Whether the runtime overlaps the two directions is
    # not under the application's control (the same process measured them at
    # the one-way rate and at up to 97 GB/s together), so the schedule is
    # given at full overlap (the best bidirectional rate measured in this run:
    # the step's lower bound) and at no overlap (every copy at its one-way rate).
    shard_b = 4 * wl.psi
    h2d_gbs = max(r["h2d_gbs"] for r in (shard_before, shard_after, fresh_after))
    d2h_gbs = max(r["d2h_gbs"] for r in (shard_before, shard_after, fresh_after))
    best_bidir = max(r["bidir_gbs"] for r in (shard_before, shard_after, fresh_after))
    d2h_s, h2d_s = shard_b / (d2h_gbs * 1e9), shard_b / (h2d_gbs * 1e9)
    bidir_s = 2 * shard_b / (best_bidir * 1e9)
    sched_ms = 1e3 * (d2h_s + (M - 1) * bidir_s + h2d_s)
    sched_fused_ms = 1e3 * (d2h_s + (M - 2) * bidir_s + h2d_s)
    serial_ms = 1e3 * (M * d2h_s + M * h2d_s)
    serial_fused_ms = 1e3 * ((M - 1) * d2h_s + (M - 1) * h2d_s)
    out = _base(wl.description, wl.psi / (ms_step * 1e-3), ms_step, args,
                {"params": wl.psi, "n_ranks": n, "chunk": C, "micro_batches": M,
                 "step": "M x chunks: reduce into slot c%2 (+H2D of the host chunk from mb 2) and D2H; "
                         "then per chunk H2D + owner Adam"})
    achieved = link_bytes / (ms_step * 1e-3) / 1e9
    out.update({
        "bound": "host link (PCIe)",
        "link_gbs": achieved,
        "link_bytes_per_step": link_bytes,
        "pinned_copy_rates_on_shard_before_steps": shard_before,
        "pinned_copy_rates_on_shard_after_steps": shard_after,
        "pinned_copy_rates_fresh_buffers_after_steps": fresh_after,
        "numa_placement": placement,
        "step_ms_each": step_ms,
        "schedule_ms_full_overlap": sched_ms,
        "schedule_ms_no_overlap": serial_ms,
        "frac_of_full_overlap_bound": sched_ms / ms_step,
        "overlap_achieved": (serial_ms - ms_step) / (serial_ms - sched_ms),
        "overlap_achieved_note": ("where the step lies between the schedule with no overlap of the two copy "
                                  "directions (0) and with full overlap at the best bidirectional rate (1)"),
        "fused_last_micro_batch": {"ms_per_step": ms_fused, "value": wl.psi / (ms_fused * 1e-3),
                                   "link_bytes_per_step": link_fused,
                                   "link_gbs": link_fused / (ms_fused * 1e-3) / 1e9,
                                   "schedule_ms_full_overlap": sched_fused_ms,
                                   "schedule_ms_no_overlap": serial_fused_ms,
                                   "frac_of_full_overlap_bound": sched_fused_ms / ms_fused},
        "roofline": {"bound": "link", "achieved": achieved, "peak": best_bidir, "unit": "GB/s",
                     "frac": achieved / best_bidir, "traffic": None,
                     "kernel": "pinned copies (both directions)",
                     "peak_note": "the best bidirectional pinned-copy rate measured in this run"},
    })
    st.engine.close()
    return out


def run_copy_calibration(args):
    """Plain copies of known size for scaling the HBM byte counters, three
    independent ones: the library's gather kernel with one 1 GiB shard, the
    runtime's device-to-device copy (torch copy_ of a contiguous tensor, which
    is hipMemcpyAsync), and a torch element-wise kernel (x * 1 over 2^28
    float32 values).  Each reads 1 GiB and writes 1 GiB per launch."""
    import torch

    import zero_sharded_optimizer_reduce_amd as z

    nbytes = 1 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    srcf, dstf = src.view(torch.float32), dst.view(torch.float32)
    T = Timer()
    res = {"calibration": "copy", "bytes_read_per_launch": nbytes, "bytes_written_per_launch": nbytes,
           "launches_each": args.steps + args.warmup}
    for name, fn in (("library_gather_kernel", lambda: z.zero_all_gather_layer([src], dst)),
                     ("runtime_device_to_device_copy", lambda: dst.copy_(src)),
                     ("torch_elementwise_mul", lambda: torch.mul(srcf, 1.0, out=dstf))):
        for _ in range(args.warmup):
            fn()
        for _ in range(args.steps):
            a = T.ev()
            fn()
            T.span(name, a, T.ev())
        torch.cuda.synchronize()
        ms = T.ms(name)
        res[name] = {"ms": ms, "gbs": 2 * nbytes / (ms * 1e-3) / 1e9}
    return res


RUNNERS = {
    "layer7b_weighted_adamw": run_layer7b,
    "tiny_flat_1m": run_tiny,
    "owner_share_8b_buckets": run_owner_share,
    "zero3_chain_llama8b": run_chain,
    "offload_owner_8b_two_slots": run_offload,
    "copy_calibration": run_copy_calibration,
}


def _nested(result):
    """A workload's result as an extra key of the line: without the fields the
    line itself states."""
    drop = {"metric", "unit", "n_gpus", "steps", "warmup", "higher_is_better", "scaling", "vs_baseline",
            "dtype", "data"}
    return {k: v for k, v in result.items() if k not in drop}


# The other workloads' figures carried by the default line, each from a child
# process: (steps, warmup) as functions of the line's own.
EXTRA_WORKLOADS = {
    "layer7b_weighted_adamw": lambda steps, warmup: (steps, warmup),
    "owner_share_8b_buckets": lambda steps, warmup: (steps, min(warmup, 3)),
    "offload_owner_8b_two_slots": lambda steps, warmup: (min(steps, 3), 1),
}


def _child_workload(name, args, steps=None, warmup=None):
    """Run one workload of this script in a child process and return its line
    (as an extra key).  Started before this process touches the GPU, so the
    two never use it at once and the child's buffers are its own fresh
    allocations; the child's progress lines go to stderr as they come."""
    import subprocess
    steps = args.steps if steps is None else steps
    warmup = args.warmup if warmup is None else warmup
    cmd = [sys.executable, os.path.abspath(__file__), "--workload", name, "--no-cpu-baseline",
           "--steps", str(steps), "--warmup", str(warmup)]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, text=True, timeout=900)
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    if r.returncode != 0 or not lines:
        return {"error": f"{' '.join(cmd[1:])} exited with {r.returncode}"}
    out = _nested(json.loads(lines[-1]))
    out["process"] = "a child process of this run, before this process used the GPU"
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="zero3_chain_llama8b", choices=sorted(RUNNERS))
    ap.add_argument("--cpu-baseline-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--chain-only", "--no-layer7b", dest="chain_only", action="store_true",
                    help="zero3_chain_llama8b: leave out the other workloads' figures (7B-class layer, owner "
                         "share, offload) that the line carries")
    ap.add_argument("--regather-bwd", action="store_true",
                    help="zero3_chain_llama8b: gather each unit again before its backward reduce")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (--gpus {args.gpus} requested): the ranks are "
              "simulated as buffers in one GPU's HBM and no multi-GPU path is built.", file=sys.stderr)
        sys.exit(2)
    cpu = None
    if args.workload in CPU_SAMPLES and not args.no_cpu_baseline:
        cpu = cpu_baseline(args.workload, args.cpu_baseline_seconds)    # before anything touches the GPU
    extras = {}
    if args.workload == "zero3_chain_llama8b" and not args.chain_only:
        for name, shape in EXTRA_WORKLOADS.items():
            steps, warmup = shape(args.steps, args.warmup)
            print(f"bench: {name} figures (child process)", file=sys.stderr, flush=True)
            extras[name] = _child_workload(name, args, steps, warmup)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    from zero_sharded_optimizer_reduce_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    print(f"bench: {args.workload}, {args.steps} timed steps after {args.warmup} warm-up steps",
          file=sys.stderr, flush=True)
    out = RUNNERS[args.workload](args)
    if cpu is not None:
        out["cpu_baseline"] = cpu
    out.update(extras)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
