"""GPU parity at full size, in the launch configuration bench.py times, on
sampled outputs the oracle computes on the host:

* one owner's 2.0e9-parameter share updated in 30 buckets of 2^26 (t=1000,
  wd=0.1): the first bucket, the partial last bucket and random windows;
* the ZeRO-3 chain over the 8B Llama-like model's 34 units: gathered views of
  sampled units, and reduced gradients and updated state of sampled units
  (embedding, first/middle/last layer, lm_head);
* the host-offloaded 2.0e9-parameter gradient shard through two slots over 4
  micro-batches: windows of the first, the partial last and random chunks.

Inputs are drawn on the device with keyed generators (synthetic.fill) and the
checked regions are copied to the host (or regenerated from their keys)."""
import gc

import numpy as np
import pytest
import torch

import oracle
import synthetic as S
from gpu_helpers import assert_grad_exact, assert_state_close, bf16_to_host, f32_to_host
from synthetic import fill
from synthetic.workloads import BUCKET, CHAIN_8B, OFFLOAD_8B, OWNER_8B

pytestmark = pytest.mark.gpu

import zero_sharded_optimizer_reduce_amd as z  # noqa: E402  (a broken package must fail, not skip)
from zero_sharded_optimizer_reduce_amd.drivers import BucketedOwnerStep, OffloadStep, Zero3Chain  # noqa: E402

W = 1 << 16     # window width


def _sc(hp):
    return oracle.adam_scalars(hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"], hp["step"])


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_owner_share_buckets_full_size():
    wl = OWNER_8B
    n = wl.n_ranks
    st = BucketedOwnerStep(wl.psi, n, BUCKET, device="cuda")
    gen = S.DeviceGen(wl.seed)
    tmp = torch.empty(BUCKET, dtype=torch.float32, device="cuda")
    fill.fill_owner_share(gen, wl, st.master, st.exp_avg, st.exp_avg_sq, st.contrib, tmp)
    del tmp
    nb = len(st.bounds)
    assert nb == 30 and st.bounds[-1][1] - st.bounds[-1][0] == wl.psi - 29 * BUCKET
    rng = np.random.default_rng(wl.seed)
    regions = [st.bounds[0], st.bounds[-1]]                      # whole first and last buckets
    for b in rng.choice(np.arange(1, nb - 1), 3, replace=False):
        lo = st.bounds[b][0] + int(rng.integers(0, BUCKET - W))
        regions.append((lo, lo + W))
    w = z.zero_rank_weights(None, n)
    hp = wl.hparams(step=wl.step0)
    pre = []
    for lo, hi in regions:
        print(f"owner share: region [{lo}, {hi})", flush=True)
        g = [bf16_to_host(c[lo:hi]) for c in st.contrib]
        pre.append((g, f32_to_host(st.master[lo:hi]), f32_to_host(st.exp_avg[lo:hi]),
                    f32_to_host(st.exp_avg_sq[lo:hi])))
        # the reduced gradient of the region, bit-exact (reduce is pure)
        red = torch.empty(hi - lo, dtype=torch.float32, device="cuda")
        z.zero_reduce_scatter([c[lo:hi] for c in st.contrib], w, [red])
        assert_grad_exact(f32_to_host(red), oracle.reduce_full(g, w), f"region {lo}")
    # the inputs were drawn from keys: regenerating one region gives the same values
    lo, hi = regions[2]
    assert np.array_equal(f32_to_host(fill.owner_share_region(gen, wl, "v", lo, hi)), pre[2][3])
    st.step(w, hp)
    torch.cuda.synchronize()
    sc = _sc(hp)
    for (lo, hi), (g, p, m, v) in zip(regions, pre):
        ref = oracle.adam_step(p, m, v, oracle.reduce_full(g, w), sc)
        assert_state_close(f32_to_host(st.master[lo:hi]), f32_to_host(st.exp_avg[lo:hi]),
                           f32_to_host(st.exp_avg_sq[lo:hi]), bf16_to_host(st.bf16[lo:hi]), ref,
                           f"region [{lo}, {hi})")


def _unit_windows(pad, s, n, rng):
    starts = {0, pad - W}
    for k in range(1, n):
        starts.add(k * s - W // 2)                 # straddles an owner boundary
    starts.update(int(x) for x in rng.integers(0, pad - W, 2))
    return sorted(starts)


def _owner_pieces(a, s):
    """Split the unit window [a, a+W) into (owner k, [j0, j1) in k's shard,
    offset of the piece inside the window)."""
    out, pos = [], a
    while pos < a + W:
        k, j0 = pos // s, pos % s
        j1 = min(s, j0 + (a + W - pos))
        out.append((k, j0, j1, pos - a))
        pos += j1 - j0
    return out


def test_zero3_chain_full_size():
    wl = CHAIN_8B
    n = wl.n_ranks
    ch = Zero3Chain(wl.extra["units"], n, device="cuda")
    assert sum(u[1] for u in ch.units) == wl.psi == 8_029_995_008
    gen = S.DeviceGen(wl.seed)
    for k in range(n):
        fill.fill_normal_pieces(gen, ch.master[k], wl.master_sigma, fill.K_MASTER + 100 * k)
        for lo, hi in fill.pieces(ch.owner_numel):
            ch.bf16[k][lo:hi].copy_(ch.master[k][lo:hi])
    U = len(ch.units)
    sampled = [0, 1, 16, U - 2, U - 1]
    rng = np.random.default_rng(wl.seed)
    wins, pre = {}, {}
    for u in sampled:
        _, psi, pad, s = ch.units[u]
        off = ch.offsets[u]
        wins[u] = _unit_windows(pad, s, n, rng)
        pre[u] = [np.concatenate([f32_to_host(ch.master[k][off + j0: off + j1])
                                  for k, j0, j1, _ in _owner_pieces(a, s)]) for a in wins[u]]
    w = z.zero_rank_weights(None, n)
    hp = wl.hparams(step=1)
    tmp = torch.empty(ch.max_pad, dtype=torch.float32, device="cuda")
    # forward: gather each unit into the temporary view, check sampled views, release
    for u in range(U):
        view = ch.forward_unit(u)
        if u in sampled:
            _, psi, pad, s = ch.units[u]
            off = ch.offsets[u]
            torch.cuda.synchronize()
            for a in wins[u]:
                exp = oracle.all_gather([bf16_to_host(ch.bf16[k][off + j0: off + j1])
                                         for k, j0, j1, _ in _owner_pieces(a, s)])
                assert np.array_equal(bf16_to_host(view[a:a + W]), exp), (u, a)
    # backward in reverse order
    sc = _sc(hp)
    for u in reversed(range(U)):
        pad = ch.units[u][2]
        fill.chain_unit_grads(gen, wl, u, ch.grads, pad, tmp)
        ch.backward_unit(u, w, hp)
        if u not in sampled:
            continue
        print(f"chain: checking unit {u}", flush=True)
        torch.cuda.synchronize()
        _, psi, pad, s = ch.units[u]
        off = ch.offsets[u]
        for a, p0 in zip(wins[u], pre[u]):
            g = [bf16_to_host(x[a:a + W]) for x in ch.grads]
            red = oracle.reduce_full(g, w)
            z0 = np.zeros(W, np.float32)
            ref = oracle.adam_step(p0, z0, z0.copy(), red, sc)
            parts = _owner_pieces(a, s)
            gpu_red = np.concatenate([f32_to_host(ch.grad_shards[k][j0:j1]) for k, j0, j1, _ in parts])
            assert_grad_exact(gpu_red, red, f"unit {u} window {a}")
            got = [np.concatenate([f32_to_host(x[k][off + j0: off + j1]) for k, j0, j1, _ in parts])
                   for x in (ch.master, ch.exp_avg, ch.exp_avg_sq)]
            got_b = np.concatenate([bf16_to_host(ch.bf16[k][off + j0: off + j1]) for k, j0, j1, _ in parts])
            assert_state_close(*got, got_b, ref, f"unit {u} window {a}")


@pytest.mark.parametrize("fuse_last", [False, True])
def test_offload_full_size(fuse_last):
    wl = OFFLOAD_8B
    n, M, C = wl.n_ranks, wl.extra["micro_batches"], wl.extra["chunk"]
    st = OffloadStep(wl.psi, n, C, device="cuda")
    gen = S.DeviceGen(wl.seed)
    tmp = torch.empty(C, dtype=torch.float32, device="cuda")
    fill.fill_normal_pieces(gen, st.master, wl.master_sigma, fill.K_MASTER)
    nc = st.n_chunks
    assert nc == 30
    rng = np.random.default_rng(wl.seed)
    chunks = [0, nc - 1] + [int(c) for c in rng.choice(np.arange(1, nc - 1), 3, replace=False)]
    wins = {}
    p0 = {}
    for c in chunks:
        L = st.chunk_len(c)
        wins[c] = sorted({0, L - W, int(rng.integers(0, L - W))})
        p0[c] = [f32_to_host(st.master[c * C + a: c * C + a + W]) for a in wins[c]]
    w = np.full(n, 1.0 / (n * M), np.float32)
    hp = wl.hparams(step=1)

    def produce(mb, c, views):
        fill.offload_contrib(gen, wl, mb, c, views, tmp)

    st.step(produce, M, w, hp, fuse_last=fuse_last)
    st.sync()
    torch.cuda.synchronize()
    host = st.host.numpy()
    sc = _sc(hp)
    bufs = [torch.empty(C, dtype=torch.bfloat16, device="cuda") for _ in range(n)]
    for c in chunks:
        print(f"offload: checking chunk {c}", flush=True)
        L = st.chunk_len(c)
        per_mb = []
        for mb in range(M):
            fill.offload_contrib(gen, wl, mb, c, [b[:L] for b in bufs], tmp)
            per_mb.append([bf16_to_host(b[:L]) for b in bufs])
        for a, p in zip(wins[c], p0[c]):
            acc = oracle.offload_accumulate([[g[a:a + W] for g in mbg] for mbg in per_mb], w)
            lo = c * C + a
            on_host = oracle.offload_accumulate([[g[a:a + W] for g in mbg] for mbg in per_mb[:M - 1]], w) \
                if fuse_last else acc
            assert_grad_exact(host[lo:lo + W], on_host, f"host shard chunk {c} window {a}")
            z0 = np.zeros(W, np.float32)
            ref = oracle.adam_step(p, z0, z0.copy(), acc, sc)
            assert_state_close(f32_to_host(st.master[lo:lo + W]), f32_to_host(st.exp_avg[lo:lo + W]),
                               f32_to_host(st.exp_avg_sq[lo:lo + W]), bf16_to_host(st.bf16[lo:lo + W]), ref,
                               f"chunk {c} window {a}")
    st.engine.close()
