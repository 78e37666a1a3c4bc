"""GPU parity at full size, in the launch configuration bench.py times, every
element of every output compared with the oracle recomputed on the host (the
reduced gradients bit for bit, the state at ulp distance 0):

* one owner's 2.0e9-parameter share updated in 30 buckets of 2^26 (t=1000,
  wd=0.1): every bucket, the partial last one included;
* one step of the ZeRO-3 chain over the 8B Llama-like model's 34 units:
  every gathered view, and every unit's reduced gradients and updated state;
* the host-offloaded 2.0e9-parameter gradient shard through two slots over 4
  micro-batches: every chunk, the partial last one included, both the host
  accumulation and the updated state.

Inputs are drawn on the device with keyed generators (synthetic.fill); each
unit, bucket or chunk is copied to the host (or its inputs regenerated from
their keys) just before or after the GPU updates it, so host memory holds one
at a time."""
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
    # the inputs were drawn from keys: regenerating one bucket gives the same values
    lo, hi = st.bounds[7]
    assert torch.equal(fill.owner_share_region(gen, wl, "v", lo, hi), st.exp_avg_sq[lo:hi])
    w = z.zero_rank_weights(None, n)
    hp = wl.hparams(step=wl.step0)
    sc = _sc(hp)
    worst = ((0, 0, 0), 0)
    # the step bucket by bucket (step() is this loop): each bucket's inputs are
    # taken just before its update, its reduced gradient from the step's own
    # bucket buffer just after
    for b in range(nb):
        lo, hi = st.bounds[b]
        g = [bf16_to_host(c[lo:hi]) for c in st.contrib]
        p, m, v = (f32_to_host(x[lo:hi]) for x in (st.master, st.exp_avg, st.exp_avg_sq))
        st.step_bucket(b, w, hp)
        torch.cuda.synchronize()
        gpu_red = f32_to_host(st.grad_bucket[: hi - lo])
        got = (f32_to_host(st.master[lo:hi]), f32_to_host(st.exp_avg[lo:hi]), f32_to_host(st.exp_avg_sq[lo:hi]),
               bf16_to_host(st.bf16[lo:hi]))

        def work(a, e):
            red = oracle.reduce_full([x[a:e] for x in g], w)
            assert_grad_exact(gpu_red[a:e], red, f"bucket {b} [{a}, {e})")
            ref = oracle.adam_step(p[a:e], m[a:e], v[a:e], red, sc)
            return assert_state_close(*(x[a:e] for x in got), ref, f"bucket {b} [{a}, {e})")

        u = max_ulps(chunked(hi - lo, work))
        worst = max_ulps([worst, u])
        print(f"owner share: bucket {b} [{lo}, {hi}): max ulp {u}", flush=True)
        del g, p, m, v, gpu_red, got
    print(f"owner share: all {nb} buckets, {wl.psi} elements, max ulp {worst}", flush=True)


CHAIN_GROUPS = 5   # the backward's 34 units in 5 tests of 6-7 units each, in backward order


@pytest.fixture(scope="module")
def chain8b():
    """The 8B chain's buffers (112 GB of owner state), filled once for the
    forward test and the backward groups of this module."""
    wl = CHAIN_8B
    n = wl.n_ranks
    ch = Zero3Chain(wl.extra["units"], n, device="cuda")
    assert sum(u[1] for u in ch.units) == wl.psi == 8_029_995_008
    gen = S.DeviceGen(wl.seed)
    for k in range(n):
        fill.fill_normal_pieces(gen, ch.master[k], wl.master_sigma, fill.K_MASTER + 100 * k)
        for lo, hi in fill.pieces(ch.owner_numel):
            ch.bf16[k][lo:hi].copy_(ch.master[k][lo:hi])
    yield ch, gen
    del ch
    gc.collect()
    torch.cuda.empty_cache()


def _unit_flat(ch, bufs, u, host=f32_to_host):
    """Unit u of per-owner buffers as one flat array in owner order."""
    s, off = ch.units[u][3], ch.offsets[u]
    return np.concatenate([host(b[off:off + s]) for b in bufs])


def test_zero3_chain_full_size_forward(chain8b):
    """Forward: every unit gathered into the temporary view, checked, released."""
    ch, _ = chain8b
    n, U = ch.n, len(ch.units)
    for u in range(U):
        view = ch.forward_unit(u)
        torch.cuda.synchronize()
        assert np.array_equal(bf16_to_host(view), oracle.all_gather(
            [bf16_to_host(ch.bf16[k][ch.offsets[u]:ch.offsets[u] + ch.units[u][3]]) for k in range(n)])), u
    print(f"chain: all {U} gathered views equal the concatenated owner shards", flush=True)


@pytest.mark.parametrize("group", range(CHAIN_GROUPS))
def test_zero3_chain_full_size_backward(chain8b, group):
    """Backward, units in reverse order (this group's share of them): every
    unit's reduced gradients and updated state, each unit's master taken just
    before its update (m = v = 0 before the first step)."""
    ch, gen = chain8b
    wl = CHAIN_8B
    n, U = ch.n, len(ch.units)
    order = list(reversed(range(U)))
    per = -(-U // CHAIN_GROUPS)
    units = order[group * per:(group + 1) * per]
    w = z.zero_rank_weights(None, n)
    hp = wl.hparams(step=1)
    sc = _sc(hp)
    tmp = torch.empty(ch.max_pad, dtype=torch.float32, device="cuda")
    worst = ((0, 0, 0), 0)
    for u in units:
        pad, s = ch.units[u][2], ch.units[u][3]
        p0 = _unit_flat(ch, ch.master, u)
        fill.chain_unit_grads(gen, wl, u, ch.grads, pad, tmp)
        ch.backward_unit(u, w, hp)
        torch.cuda.synchronize()
        g = [bf16_to_host(x[:pad]) for x in ch.grads]
        gpu_red = np.concatenate([f32_to_host(x[:s]) for x in ch.grad_shards])
        got = tuple(_unit_flat(ch, b, u) for b in (ch.master, ch.exp_avg, ch.exp_avg_sq)) + \
            (_unit_flat(ch, ch.bf16, u, bf16_to_host),)

        def work(a, e):
            red = oracle.reduce_full([x[a:e] for x in g], w)
            assert_grad_exact(gpu_red[a:e], red, f"unit {u} [{a}, {e})")
            z0 = np.zeros(e - a, np.float32)
            ref = oracle.adam_step(p0[a:e], z0, z0.copy(), red, sc)
            return assert_state_close(*(x[a:e] for x in got), ref, f"unit {u} [{a}, {e})")

        ulps = max_ulps(chunked(pad, work))
        worst = max_ulps([worst, ulps])
        print(f"chain: unit {u} ({ch.units[u][0]}): {pad} elements, max ulp {ulps}", flush=True)
        del g, gpu_red, got, p0
    print(f"chain: units {units[0]}..{units[-1]}, max ulp {worst}", flush=True)


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
    p0 = f32_to_host(st.master)                    # m = v = 0 before the first step
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
    worst = ((0, 0, 0), 0)
    for c in range(nc):
        L, base = st.chunk_len(c), c * C
        per_mb = []
        for mb in range(M):
            fill.offload_contrib(gen, wl, mb, c, [b[:L] for b in bufs], tmp)
            per_mb.append([bf16_to_host(b[:L]) for b in bufs])
        got = tuple(f32_to_host(x[base:base + L]) for x in (st.master, st.exp_avg, st.exp_avg_sq)) + \
            (bf16_to_host(st.bf16[base:base + L]),)
        p = p0[base:base + L]

        def work(a, e):
            acc = oracle.offload_accumulate([[g[a:e] for g in mbg] for mbg in per_mb], w)
            on_host = oracle.offload_accumulate([[g[a:e] for g in mbg] for mbg in per_mb[:M - 1]], w) \
                if fuse_last else acc
            assert_grad_exact(host[base + a:base + e], on_host, f"host shard chunk {c} [{a}, {e})")
            z0 = np.zeros(e - a, np.float32)
            ref = oracle.adam_step(p[a:e], z0, z0.copy(), acc, sc)
            return assert_state_close(*(x[a:e] for x in got), ref, f"chunk {c} [{a}, {e})")

        ulps = max_ulps(chunked(L, work))
        worst = max_ulps([worst, ulps])
        print(f"offload (fuse_last={fuse_last}): chunk {c}: {L} elements, max ulp {ulps}", flush=True)
        del per_mb, got
    print(f"offload (fuse_last={fuse_last}): all {nc} chunks, {wl.psi} elements, max ulp {worst}", flush=True)
    st.engine.close()
