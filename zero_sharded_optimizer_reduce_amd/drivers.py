"""Step drivers: sequence the C-ABI calls for one ZeRO step over N simulated
ranks whose buffers all live in one GPU's HBM.  Orchestration only; every
arithmetic step runs in the HIP kernels of libzero.

* ShardedStep       flat unit: reduce-scatter -> N owner updates -> all-gather
                    (blog "数据并行与 ZeRO：三级分片各省多少", section 三级分片,
                    ZeRO-1/2 paragraphs; slide "分担数据，与分担保存责任，是两个
                    动作", note 原 N48)
* BucketedOwnerStep one owner's share in fixed-size gradient buckets (essay
                    "把训练账本放进多张设备", section ZeRO-3 的一次完整计算,
                    bucketing paragraph)
* Zero3Chain        per-layer gather/release forward, reverse-order reduce and
                    update backward (essay, section ZeRO-3 的一次完整计算;
                    slide, note 原 N47)
* OffloadStep       host-resident gradient shard through two device slots (blog,
                    section 分片放到 CPU：两个缓冲就够)
* GraphedStep       a ShardedStep captured once into a HIP graph and replayed
                    every step, the step's Adam scalars read from device memory
"""
from __future__ import annotations

from typing import Optional, Sequence

import torch

from .api import (ADAM_SCALARS_FLOATS, ZeroOffload, adam_scalars_tensor, zero_adam_scalars_fetch,
                  zero_adam_shard_step, zero_adam_shard_step_dev, zero_all_gather_layer, zero_reduce_scatter,
                  zero_reduce_scatter_adam, zero_reduce_scatter_adam_dev, zero_shard_layout)


def _empty(n, dtype, device):
    return torch.empty(int(n), dtype=dtype, device=device)


class ShardedStep:
    """One flat unit of psi parameters, padded to psi_pad and split into N owner
    shards.  Owner k holds FP32 master/m/v and its BF16 working shard; the
    reduced FP32 gradient shards are transient step buffers."""

    def __init__(self, numels: Sequence[int], n_ranks: int, device="cuda"):
        self.n = n_ranks
        self.psi, self.psi_pad, self.shard = zero_shard_layout(list(numels), n_ranks)
        self.device = torch.device(device)
        S = self.shard
        self.master = [_empty(S, torch.float32, device) for _ in range(n_ranks)]
        self.exp_avg = [torch.zeros(S, dtype=torch.float32, device=device) for _ in range(n_ranks)]
        self.exp_avg_sq = [torch.zeros(S, dtype=torch.float32, device=device) for _ in range(n_ranks)]
        self.bf16 = [_empty(S, torch.bfloat16, device) for _ in range(n_ranks)]
        self.grad = [_empty(S, torch.float32, device) for _ in range(n_ranks)]
        self.view = _empty(self.psi_pad, torch.bfloat16, device)

    def load_master(self, flat_master: torch.Tensor) -> None:
        """Set the owners' masters from a padded flat FP32 vector."""
        for k in range(self.n):
            self.master[k].copy_(flat_master[k * self.shard:(k + 1) * self.shard])

    def reduce_scatter(self, rank_grads, weights, stream=None):
        zero_reduce_scatter(rank_grads, weights, self.grad, stream=stream)

    def update(self, hp, stream=None):
        for k in range(self.n):
            zero_adam_shard_step(self.master[k], self.exp_avg[k], self.exp_avg_sq[k], self.bf16[k],
                                 self.grad[k], hp, stream=stream)

    def all_gather(self, stream=None):
        zero_all_gather_layer(self.bf16, self.view, stream=stream)

    def step(self, rank_grads, weights, hp, stream=None):
        self.reduce_scatter(rank_grads, weights, stream)
        self.update(hp, stream)
        self.all_gather(stream)
        return self.view[: self.psi]


class GraphedStep:
    """A ShardedStep captured once into a HIP graph (torch.cuda.CUDAGraph) and
    replayed at every step: reduce-scatter, the owners' updates, all-gather
    (or the fused reduce + update storing the reduced shards, then the
    all-gather).  The updates read the step's scalars from a device struct
    that the graph's first kernel (zero_adam_scalars_fetch) fills from a ring
    of pinned host slots, taking the next slot at every replay; step() writes
    this step's scalars into that slot and replays, with no copy call between
    replays.  Results are bit-identical to ShardedStep.step with the same
    hyper-parameters.  The caller writes each step's contributions into the
    captured rank_grads buffers; the rank weights are those of the capture.
    A slot is rewritten only after the replay that read it has completed."""

    RING = 8          # ring slots: a power of two, as the fetch kernel requires
    EVENT_EVERY = 4   # replays per completion event (RING // 2)

    def __init__(self, st: ShardedStep, rank_grads, weights, fused: bool = False):
        self.st = st
        self.rank_grads = list(rank_grads)
        dev = st.device
        self.scalars = torch.zeros(ADAM_SCALARS_FLOATS, dtype=torch.float32, device=dev)
        self.cursor = torch.zeros(1, dtype=torch.int32, device=dev)
        self.ring = torch.zeros(self.RING, ADAM_SCALARS_FLOATS, dtype=torch.float32, pin_memory=True)
        self._events = {}   # group of EVENT_EVERY replays -> event recorded after its last replay
        self._t = 0
        self.graph = torch.cuda.CUDAGraph()
        torch.cuda.synchronize(dev)
        with torch.cuda.graph(self.graph):
            zero_adam_scalars_fetch(self.ring, self.cursor, self.scalars)
            if fused:
                zero_reduce_scatter_adam_dev(self.rank_grads, weights, st.master, st.exp_avg, st.exp_avg_sq,
                                             st.bf16, self.scalars, grad_out=st.grad)
            else:
                zero_reduce_scatter(self.rank_grads, weights, st.grad)
                for k in range(st.n):
                    zero_adam_shard_step_dev(st.master[k], st.exp_avg[k], st.exp_avg_sq[k], st.bf16[k],
                                             st.grad[k], self.scalars)
            zero_all_gather_layer(st.bf16, st.view)
        torch.cuda.synchronize(dev)

    def step(self, hp):
        """One step on the current stream: this step's scalars into its ring
        slot, then the replay.  Slot t mod RING was last read by replay
        t - RING.  At the first step of each group of EVENT_EVERY steps the
        host waits for the event recorded after replay t - RING +
        EVENT_EVERY - 1, which frees the slots of this step and of the next
        EVENT_EVERY - 1 steps; the host stays up to RING - EVENT_EVERY + 1
        replays ahead of the device."""
        t = self._t
        if t >= self.RING and (t - self.RING) % self.EVENT_EVERY == 0:
            self._events.pop((t - self.RING) // self.EVENT_EVERY).synchronize()
        adam_scalars_tensor(hp, out=self.ring[t % self.RING])
        self.graph.replay()
        if t % self.EVENT_EVERY == self.EVENT_EVERY - 1:
            ev = torch.cuda.Event()
            ev.record()
            self._events[t // self.EVENT_EVERY] = ev
        self._t = t + 1
        return self.st.view[: self.st.psi]


class BucketedOwnerStep:
    """One owner's share of S parameters updated bucket by bucket: for each
    bucket the N pre-sliced contributions are reduced into one reused FP32
    bucket buffer, then the owner's state slice is updated from it."""

    def __init__(self, shard_numel: int, n_ranks: int, bucket: int, device="cuda",
                 allocate_state: bool = True):
        self.S, self.n, self.bucket = int(shard_numel), n_ranks, int(bucket)
        self.device = torch.device(device)
        self.bounds = [(lo, min(lo + self.bucket, self.S)) for lo in range(0, self.S, self.bucket)]
        self.grad_bucket = _empty(min(self.bucket, self.S), torch.float32, device)
        if allocate_state:
            self.master = _empty(self.S, torch.float32, device)
            self.exp_avg = _empty(self.S, torch.float32, device)
            self.exp_avg_sq = _empty(self.S, torch.float32, device)
            self.bf16 = _empty(self.S, torch.bfloat16, device)
            self.contrib = [_empty(self.S, torch.bfloat16, device) for _ in range(n_ranks)]

    def step_bucket(self, b: int, weights, hp, stream=None):
        lo, hi = self.bounds[b]
        g = self.grad_bucket[: hi - lo]
        zero_reduce_scatter([c[lo:hi] for c in self.contrib], weights, [g], stream=stream)
        zero_adam_shard_step(self.master[lo:hi], self.exp_avg[lo:hi], self.exp_avg_sq[lo:hi],
                             self.bf16[lo:hi], g, hp, stream=stream)

    def step(self, weights, hp, stream=None):
        for b in range(len(self.bounds)):
            self.step_bucket(b, weights, hp, stream)


class Zero3Chain:
    """ZeRO-3 per-unit chain: every unit's weights live only as N BF16 owner
    shards (plus FP32 master/m/v per owner).  Forward: for each unit in order,
    all-gather the shards into a temporary full view, then release it.
    Backward: for each unit in reverse order, the caller writes the unit's N
    BF16 gradient contributions into `grads` (the first units[u][2] elements
    of each: the unit's padded length); they are reduce-scattered and applied
    by each owner's update."""

    def __init__(self, units, n_ranks: int, device="cuda"):
        self.n = n_ranks
        self.device = torch.device(device)
        self.units = []
        for name, tensors in units:
            psi, pad, s = zero_shard_layout([t for _, t in tensors], n_ranks)
            self.units.append((name, psi, pad, s))
        self.max_pad = max(u[2] for u in self.units)
        self.max_shard = max(u[3] for u in self.units)
        # per-owner flat state, unit u at offset self.offsets[u] within each owner buffer
        self.offsets, off = [], 0
        for _, _, _, s in self.units:
            self.offsets.append(off)
            off += s
        self.owner_numel = off
        n = n_ranks
        self.master = [_empty(off, torch.float32, device) for _ in range(n)]
        self.exp_avg = [torch.zeros(off, dtype=torch.float32, device=device) for _ in range(n)]
        self.exp_avg_sq = [torch.zeros(off, dtype=torch.float32, device=device) for _ in range(n)]
        self.bf16 = [_empty(off, torch.bfloat16, device) for _ in range(n)]
        # transient per-step buffers, sized for the largest unit
        self.grads = [_empty(self.max_pad, torch.bfloat16, device) for _ in range(n)]
        self.grad_shards = [_empty(self.max_shard, torch.float32, device) for _ in range(n)]
        self.view = None

    def owner_slices(self, u: int, bufs):
        s, off = self.units[u][3], self.offsets[u]
        return [b[off:off + s] for b in bufs]

    def forward_unit(self, u: int, stream=None, release: bool = True):
        pad = self.units[u][2]
        if self.view is None:
            self.view = _empty(self.max_pad, torch.bfloat16, self.device)
        view = self.view[:pad]
        zero_all_gather_layer(self.owner_slices(u, self.bf16), view, stream=stream)
        return view

    def backward_unit_fused(self, u: int, weights, hp, stream=None, regather: bool = False):
        """backward_unit with the fused reduce-scatter + update kernel (one
        launch per owner; the reduced shards are not stored)."""
        pad = self.units[u][2]
        if regather:
            self.forward_unit(u, stream=stream)
        zero_reduce_scatter_adam([g[:pad] for g in self.grads], weights,
                                 *(self.owner_slices(u, x) for x in
                                   (self.master, self.exp_avg, self.exp_avg_sq, self.bf16)),
                                 hp, stream=stream)

    def backward_unit(self, u: int, weights, hp, stream=None, regather: bool = False):
        """Reduce-scatter unit u's N contributions into the owners' FP32
        gradient shards, then each owner's update.  With regather, the unit's
        weights are first gathered again into the view, as the backward pass
        needs them (essay, ZeRO-3 的一次完整计算: backward gathers each layer
        again before computing its gradient)."""
        if regather:
            self.forward_unit(u, stream=stream)
        self.reduce_unit(u, weights, stream=stream)
        self.update_unit(u, hp, stream=stream)

    def reduce_unit(self, u: int, weights, stream=None):
        """Unit u's N contributions reduce-scattered into the owners' FP32
        gradient shards."""
        pad, s = self.units[u][2], self.units[u][3]
        zero_reduce_scatter([g[:pad] for g in self.grads], weights,
                            [g[:s] for g in self.grad_shards], stream=stream)

    def update_unit(self, u: int, hp, stream=None):
        """Each owner's update of its slice of unit u from its gradient shard."""
        s = self.units[u][3]
        for k, (p, m, v, b) in enumerate(zip(*(self.owner_slices(u, x) for x in
                                              (self.master, self.exp_avg, self.exp_avg_sq, self.bf16)))):
            zero_adam_shard_step(p, m, v, b, self.grad_shards[k][:s], hp, stream=stream)


class OffloadStep:
    """One owner's shard of S parameters whose FP32 gradient accumulator lives in
    pinned host memory; the device holds two chunk slots of N BF16
    contributions and two FP32 staging chunks, plus the owner's master/m/v and
    BF16 working shard."""

    def __init__(self, shard_numel: int, n_ranks: int, chunk: int, device="cuda"):
        self.S, self.n, self.chunk = int(shard_numel), n_ranks, int(chunk)
        self.device = torch.device(device)
        self.host = torch.empty(self.S, dtype=torch.float32, pin_memory=True)
        self.slot_contrib = [_empty(n_ranks * self.chunk, torch.bfloat16, device) for _ in range(2)]
        self.slot_f32 = [_empty(self.chunk, torch.float32, device) for _ in range(2)]
        self.master = _empty(self.S, torch.float32, device)
        self.exp_avg = torch.zeros(self.S, dtype=torch.float32, device=device)
        self.exp_avg_sq = torch.zeros(self.S, dtype=torch.float32, device=device)
        self.bf16 = _empty(self.S, torch.bfloat16, device)
        self.engine = ZeroOffload(n_ranks, self.S, self.chunk, self.host, self.slot_contrib, self.slot_f32)
        self.n_chunks = self.engine.n_chunks

    def chunk_len(self, c: int) -> int:
        return self.engine.chunk_len(c)

    def contrib_views(self, c: int):
        """The N rank contribution views of chunk c inside its slot."""
        slot = self.slot_contrib[c % 2]
        L = self.chunk_len(c)
        return [slot[r * self.chunk: r * self.chunk + L] for r in range(self.n)]

    def step(self, produce, n_micro: int, weights, hp, stream=None, fuse_last: bool = False):
        """produce(mb, c, views) writes chunk c's contributions for micro-batch
        mb into `views` on the current stream.  fuse_last: the last
        micro-batch's reduction is applied directly (REDUCE_ADAM) instead of
        going to the host and streaming back (ADAM)."""
        for mb in range(n_micro):
            last = fuse_last and mb == n_micro - 1
            for c in range(self.n_chunks):
                produce(mb, c, self.contrib_views(c))
                if last:
                    self.engine.reduce_adam(c, mb, weights, self.master, self.exp_avg, self.exp_avg_sq,
                                            self.bf16, hp, stream)
                else:
                    self.engine.reduce(c, mb, weights, stream)
        if not fuse_last:
            for c in range(self.n_chunks):
                self.engine.adam(c, self.master, self.exp_avg, self.exp_avg_sq, self.bf16, hp, stream)

    def sync(self):
        self.engine.sync()
