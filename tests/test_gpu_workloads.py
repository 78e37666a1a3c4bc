"""GPU parity at full size, in the launch configuration bench.py times, on
whole sampled units that the oracle recomputes on the host, every element
compared (the reduced gradients bit for bit, the state at ulp distance 0):

* one owner's 2.0e9-parameter share updated in 30 buckets of 2^26 (t=1000,
  wd=0.1): the first bucket, the partial last bucket and 3 seeded random
  buckets;
* the ZeRO-3 chain over the 8B Llama-like model's 34 units: the embedding,
  the lm_head and 3 seeded random layers: their gathered views, reduced
  gradients and updated state;
* the host-offloaded 2.0e9-parameter gradient shard through two slots over 4
  micro-batches: the first chunk, the partial last chunk and 3 seeded random
  chunks, both the host accumulation and the updated state.

Inputs are drawn on the device with keyed generators (synthetic.fill) and the
checked units are copied to the host (or regenerated from their keys)."""
import gc

import numpy as np
import pytest
import torch

import oracle
import synthetic as S
from gpu_helpers import (assert_grad_exact, assert_state_close, bf16_to_host, chunked, f32_to_host,
                         max_ulps)
from synthetic import fill
from synthetic.workloads import BUCKET, CHAIN_8B, OFFLOAD_8B, OWNER_8B

pytestmark = pytest.mark.gpu

import zero_sharded_optimizer_reduce_amd as z  # noqa: E402  (a broken package must fail, not skip)
from zero_sharded_optimizer_reduce_amd.drivers import BucketedOwnerStep, OffloadStep, Zero3Chain  # noqa: E402


def _sc(hp):
    return oracle.adam_scalars(hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"], hp["step"])


def _first_last_random(n, rng, k=3):
    """Indices 0 and n-1 and k seeded random ones between them."""
    return [0, n - 1] + sorted(int(x) for x in rng.choice(np.arange(1, n - 1), k, replace=False))


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
    picks = _first_last_random(nb, np.random.default_rng(wl.seed))
    w = z.zero_rank_weights(None, n)
    hp = wl.hparams(step=wl.step0)
    pre = {}
    for b in picks:
        lo, hi = st.bounds[b]
        print(f"owner share: bucket {b} [{lo}, {hi})", flush=True)
        # the reduced gradient of the bucket, as the step computes it (the
        # step's own bucket buffer is reused, so it is taken here)
        red = torch.empty(hi - lo, dtype=torch.float32, device="cuda")
        z.zero_reduce_scatter([c[lo:hi] for c in st.contrib], w, [red])
        pre[b] = ([bf16_to_host(c[lo:hi]) for c in st.contrib], f32_to_host(st.master[lo:hi]),
                  f32_to_host(st.exp_avg[lo:hi]), f32_to_host(st.exp_avg_sq[lo:hi]), f32_to_host(red))
        del red
    # the inputs were drawn from keys: regenerating one bucket gives the same values
    lo, hi = st.bounds[picks[2]]
    assert np.array_equal(f32_to_host(fill.owner_share_region(gen, wl, "v", lo, hi)), pre[picks[2]][3])
    st.step(w, hp)
    torch.cuda.synchronize()
    sc = _sc(hp)
    for b in picks:
        lo, hi = st.bounds[b]
        g, p, m, v, gpu_red = pre[b]
        got = (f32_to_host(st.master[lo:hi]), f32_to_host(st.exp_avg[lo:hi]), f32_to_host(st.exp_avg_sq[lo:hi]),
               bf16_to_host(st.bf16[lo:hi]))

        def work(a, e):
            red = oracle.reduce_full([x[a:e] for x in g], w)
            assert_grad_exact(gpu_red[a:e], red, f"bucket {b} [{a}, {e})")
            ref = oracle.adam_step(p[a:e], m[a:e], v[a:e], red, sc)
            return assert_state_close(*(x[a:e] for x in got), ref, f"bucket {b} [{a}, {e})")

        print(f"owner share: bucket {b}: {hi - lo} elements, max ulp {max_ulps(chunked(hi - lo, work))}", flush=True)


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
    sampled = _first_last_random(U, np.random.default_rng(wl.seed))

    def flat(bufs, u, host=f32_to_host):
        """Unit u of per-owner buffers as one flat array in owner order."""
        s, off = ch.units[u][3], ch.offsets[u]
        return np.concatenate([host(b[off:off + s]) for b in bufs])

    pre = {u: flat(ch.master, u) for u in sampled}        # m = v = 0 before the first step
    w = z.zero_rank_weights(None, n)
    hp = wl.hparams(step=1)
    tmp = torch.empty(ch.max_pad, dtype=torch.float32, device="cuda")
    # forward: gather each unit into the temporary view, check sampled views, release
    for u in range(U):
        view = ch.forward_unit(u)
        if u in sampled:
            torch.cuda.synchronize()
            print(f"chain: view of unit {u} ({ch.units[u][0]}, {ch.units[u][2]} elements)", flush=True)
            assert np.array_equal(bf16_to_host(view), oracle.all_gather(
                [bf16_to_host(ch.bf16[k][ch.offsets[u]:ch.offsets[u] + ch.units[u][3]]) for k in range(n)])), u
    # backward in reverse order
    sc = _sc(hp)
    for u in reversed(range(U)):
        pad, s = ch.units[u][2], ch.units[u][3]
        fill.chain_unit_grads(gen, wl, u, ch.grads, pad, tmp)
        ch.backward_unit(u, w, hp)
        if u not in sampled:
            continue
        torch.cuda.synchronize()
        g = [bf16_to_host(x[:pad]) for x in ch.grads]
        gpu_red = np.concatenate([f32_to_host(x[:s]) for x in ch.grad_shards])
        got = (flat(ch.master, u), flat(ch.exp_avg, u), flat(ch.exp_avg_sq, u), flat(ch.bf16, u, bf16_to_host))
        p0 = pre.pop(u)

        def work(a, e):
            red = oracle.reduce_full([x[a:e] for x in g], w)
            assert_grad_exact(gpu_red[a:e], red, f"unit {u} [{a}, {e})")
            z0 = np.zeros(e - a, np.float32)
            ref = oracle.adam_step(p0[a:e], z0, z0.copy(), red, sc)
            return assert_state_close(*(x[a:e] for x in got), ref, f"unit {u} [{a}, {e})")

        print(f"chain: unit {u} ({ch.units[u][0]}): {pad} elements, max ulp {max_ulps(chunked(pad, work))}",
              flush=True)
        del g, gpu_red, got, p0


@pytest.mark.parametrize("fuse_last", [False, True])
def test_offload_full_size(fuse_last):
    wl = OFFLOAD_8B
    n, M, C = wl.n_ranks, wl.extra["micro_batches"], wl.extra["chunk"]
    st = OffloadStep(wl.psi, n, C, device="cuda")
    gen = S.DeviceGen(wl.seed)
    tmp = torch.empty(C, dtype=torch.float32, device="cuda")
    fill.fill_normal_pieces(gen, st.master, wl.master_sigma, fill.K_MASTER)
    nc = st.n_chunks
    assert nc == 30 and st.chunk_len(nc - 1) < C
    chunks = _first_last_random(nc, np.random.default_rng(wl.seed))
    p0 = {c: f32_to_host(st.master[c * C: c * C + st.chunk_len(c)]) for c in chunks}
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
        L, base = st.chunk_len(c), c * C
        per_mb = []
        for mb in range(M):
            fill.offload_contrib(gen, wl, mb, c, [b[:L] for b in bufs], tmp)
            per_mb.append([bf16_to_host(b[:L]) for b in bufs])
        got = tuple(f32_to_host(x[base:base + L]) for x in (st.master, st.exp_avg, st.exp_avg_sq)) + \
            (bf16_to_host(st.bf16[base:base + L]),)
        p = p0[c]

        def work(a, e):
            acc = oracle.offload_accumulate([[g[a:e] for g in mbg] for mbg in per_mb], w)
            on_host = oracle.offload_accumulate([[g[a:e] for g in mbg] for mbg in per_mb[:M - 1]], w) \
                if fuse_last else acc
            assert_grad_exact(host[base + a:base + e], on_host, f"host shard chunk {c} [{a}, {e})")
            z0 = np.zeros(e - a, np.float32)
            ref = oracle.adam_step(p[a:e], z0, z0.copy(), acc, sc)
            return assert_state_close(*(x[a:e] for x in got), ref, f"chunk {c} [{a}, {e})")

        print(f"offload (fuse_last={fuse_last}): chunk {c}: {L} elements, max ulp {max_ulps(chunked(L, work))}",
              flush=True)
    st.engine.close()
