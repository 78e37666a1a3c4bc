"""GPU parity of the two-slot host-offload engine (zero_offload_*): the pinned
host shard after M micro-batches equals the oracle's accumulation, the state
after the streamed-back update equals the oracle's Adam on it, and the result
does not change when the side streams are delayed or released staging buffers
are poisoned (so a missing wait would show up as a wrong or NaN value)."""
import os

import numpy as np
import pytest
import torch

import oracle
import synthetic as S
from gpu_helpers import assert_grad_exact, assert_state_close, bf16_to_dev, bf16_to_host, f32_to_host

pytestmark = pytest.mark.gpu

import zero_sharded_optimizer_reduce_amd as z  # noqa: E402  (a broken package must fail, not skip)
from zero_sharded_optimizer_reduce_amd import _lib  # noqa: E402
from zero_sharded_optimizer_reduce_amd.drivers import OffloadStep  # noqa: E402


def _run(shard, chunk, n_ranks=4, n_micro=4, seed=0, env=None, fuse_last=False):
    env = env or {}
    old = {k: os.environ.get(k) for k in env}
    os.environ.update(env)
    try:
        st = OffloadStep(shard, n_ranks, chunk, device="cuda")
    finally:
        for k, v in old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    g = S.rng(seed)
    contrib = [[[S.bf16_normal(g, st.chunk_len(c), 1e-3) for _ in range(n_ranks)]
                for c in range(st.n_chunks)] for _ in range(n_micro)]
    pool = [[[bf16_to_dev(x) for x in rc] for rc in mb] for mb in contrib]
    p0, m0, v0 = S.host_state(seed + 1, shard, 0.02)
    st.master.copy_(torch.from_numpy(p0))
    w = np.full(n_ranks, 1.0 / (n_ranks * n_micro), np.float32)
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, step=1)

    def produce(mb, c, views):
        for r, vw in enumerate(views):
            vw.copy_(pool[mb][c][r])

    st.step(produce, n_micro, w, hp, fuse_last=fuse_last)
    st.sync()
    torch.cuda.synchronize()
    host = st.host.numpy().copy()
    sc = oracle.adam_scalars(1e-3, 0.9, 0.999, 1e-8, 0.0, 1)
    for c in range(st.n_chunks):
        lo, hi = c * chunk, c * chunk + st.chunk_len(c)
        acc = oracle.offload_accumulate([contrib[mb][c] for mb in range(n_micro)], w)
        if fuse_last:
            # the host holds micro-batches 0..M-2; the last one was applied on the device
            if n_micro > 1:
                assert_grad_exact(host[lo:hi], oracle.offload_accumulate(
                    [contrib[mb][c] for mb in range(n_micro - 1)], w), f"host chunk {c}")
        else:
            assert_grad_exact(host[lo:hi], acc, f"host chunk {c}")
        ref = oracle.adam_step(p0[lo:hi], m0[lo:hi], v0[lo:hi], acc, sc)
        assert_state_close(f32_to_host(st.master[lo:hi]), f32_to_host(st.exp_avg[lo:hi]),
                           f32_to_host(st.exp_avg_sq[lo:hi]), bf16_to_host(st.bf16[lo:hi]), ref,
                           f"chunk {c}")
    st.engine.close()


@pytest.mark.parametrize("shard,chunk", [(3 * 8192 + 1000, 8192), (8192, 8192), (5 * 1000 + 7, 1000),
                                         (1, 1 << 10), (9 * 4096, 4096)])
@pytest.mark.parametrize("fuse_last", [False, True])
def test_offload_matches_oracle(shard, chunk, fuse_last):
    print(f"offload shard={shard} chunk={chunk} fuse_last={fuse_last}", flush=True)
    _run(shard, chunk, fuse_last=fuse_last)


@pytest.mark.parametrize("fuse_last", [False, True])
def test_offload_with_delayed_side_streams_and_poison(fuse_last):
    _run(7 * 4096 + 123, 4096, env={"ZERO_OFFLOAD_DEBUG_DELAY_US": "3000",
                                    "ZERO_OFFLOAD_DEBUG_POISON": "1"}, seed=5, fuse_last=fuse_last)


@pytest.mark.parametrize("fuse_last", [False, True])
def test_offload_single_micro_batch_and_ranks(fuse_last):
    _run(4 * 2048, 2048, n_ranks=1, n_micro=1, seed=7, fuse_last=fuse_last)
    _run(4 * 2048 + 8, 2048, n_ranks=3, n_micro=2, seed=8, fuse_last=fuse_last)


def test_offload_misuse_is_rejected():
    st = OffloadStep(4 * 1024, 4, 1024, device="cuda")
    w = np.full(4, 0.25, np.float32)
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, step=1)
    for v in st.slot_contrib:
        v.zero_()
    with pytest.raises(z.ZeroError, match="ZERO_ERR_STATE"):
        st.engine.reduce(0, 1, w)                 # micro-batch 1 before micro-batch 0
    with pytest.raises(z.ZeroError, match="ZERO_ERR_STATE"):
        st.engine.adam(1, st.master, st.exp_avg, st.exp_avg_sq, st.bf16, hp)   # never reduced
    with pytest.raises(z.ZeroError, match="ZERO_ERR_STATE"):
        st.engine.reduce(4, 0, w)                 # chunk out of range
    st.engine.reduce(0, 0, w)
    st.engine.reduce(0, 1, w)
    st.engine.adam(0, st.master, st.exp_avg, st.exp_avg_sq, st.bf16, hp)
    # the update consumed chunk 0's accumulation: neither a further micro-batch
    # onto it nor a second update may follow; a new accumulation starts at 0
    with pytest.raises(z.ZeroError, match="ZERO_ERR_STATE"):
        st.engine.reduce(0, 2, w)
    with pytest.raises(z.ZeroError, match="ZERO_ERR_STATE"):
        st.engine.adam(0, st.master, st.exp_avg, st.exp_avg_sq, st.bf16, hp)
    st.engine.reduce_adam(1, 0, w, st.master, st.exp_avg, st.exp_avg_sq, st.bf16, hp)
    with pytest.raises(z.ZeroError, match="ZERO_ERR_STATE"):
        st.engine.reduce(1, 1, w)
    st.engine.reduce(0, 0, w)
    st.sync()
    st.engine.close()
    # a host shard that is not pinned and mapped for the device (the
    # device-to-host copy is a kernel writing through that mapping)
    # (called through the C ABI: the binding itself already refuses it)
    import ctypes
    pageable = torch.zeros(4 * 1024, dtype=torch.float32)
    slots = [torch.zeros(4 * 1024, dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    stage = [torch.zeros(1024, device="cuda") for _ in range(2)]
    handle = ctypes.c_void_p()
    tables = [(ctypes.c_void_p * 2)(*(t.data_ptr() for t in ts)) for ts in (slots, stage)]
    status = _lib.load().zero_offload_create(4, pageable.numel(), 1024, pageable.data_ptr(), tables[0],
                                             tables[1], ctypes.byref(handle))
    assert status == _lib.ZERO_ERR_ARG and not handle.value
    assert b"not pinned" in _lib.load().zero_last_error()
    with pytest.raises(ValueError):
        z.zero_offload_create(4, pageable.numel(), 1024, pageable, slots, stage)
    # more chunks than a handle may hold (two events per chunk)
    chunk = 16
    host = torch.zeros(_lib.ZERO_OFFLOAD_MAX_CHUNKS * chunk + 1, dtype=torch.float32, pin_memory=True)
    slots = [torch.zeros(4 * chunk, dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    stage = [torch.zeros(chunk, device="cuda") for _ in range(2)]
    with pytest.raises(z.ZeroError, match="ZERO_ERR_SIZE"):
        z.zero_offload_create(4, host.numel(), chunk, host, slots, stage)


@pytest.mark.parametrize("fuse_last_2", [False, True])
def test_offload_compute_stream_changes_between_steps(fuse_last_2):
    """Step 1 runs on stream A, its updates held back by a spin kernel; step 2
    runs on stream B, whose contribution writes wait only for step 1's
    reductions.  Step 2's first reductions write the staging slots that step
    1's delayed updates still read, so the handle itself must order them.
    Both steps are checked against the oracle (host accumulation, then the
    state after t=1 and t=2)."""
    if not hasattr(torch.cuda, "_sleep"):
        pytest.skip("torch.cuda._sleep not available")
    shard, chunk, n_ranks, n_micro = 4 * 4096 + 100, 4096, 4, 2
    print(f"offload stream change shard={shard} chunk={chunk} fuse_last_2={fuse_last_2}", flush=True)
    st = OffloadStep(shard, n_ranks, chunk, device="cuda")
    g = S.rng(11)
    contrib = [[[[S.bf16_normal(g, st.chunk_len(c), 1e-3) for _ in range(n_ranks)]
                 for c in range(st.n_chunks)] for _ in range(n_micro)] for _ in range(2)]
    pool = [[[[bf16_to_dev(x) for x in rc] for rc in mb] for mb in step] for step in contrib]
    p0, m0, v0 = S.host_state(12, shard, 0.02)
    st.master.copy_(torch.from_numpy(p0))
    w = np.full(n_ranks, 1.0 / (n_ranks * n_micro), np.float32)
    hps = [dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, step=t) for t in (1, 2)]
    A, B = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()

    def produce(step, mb, c):
        for r, vw in enumerate(st.contrib_views(c)):
            vw.copy_(pool[step][mb][c][r])

    with torch.cuda.stream(A):
        for mb in range(n_micro):
            for c in range(st.n_chunks):
                produce(0, mb, c)
                st.engine.reduce(c, mb, w, stream=A)
        reduced = torch.cuda.Event()
        reduced.record(A)
        for c in range(st.n_chunks):
            torch.cuda._sleep(20_000_000)      # bounded spin: delays this update on A
            st.engine.adam(c, st.master, st.exp_avg, st.exp_avg_sq, st.bf16, hps[0], stream=A)
    with torch.cuda.stream(B):
        B.wait_event(reduced)                  # the contribution slots are free after the reductions
        for mb in range(n_micro):
            last = fuse_last_2 and mb == n_micro - 1
            for c in range(st.n_chunks):
                produce(1, mb, c)
                if last:
                    st.engine.reduce_adam(c, mb, w, st.master, st.exp_avg, st.exp_avg_sq, st.bf16, hps[1],
                                          stream=B)
                else:
                    st.engine.reduce(c, mb, w, stream=B)
        if not fuse_last_2:
            for c in range(st.n_chunks):
                st.engine.adam(c, st.master, st.exp_avg, st.exp_avg_sq, st.bf16, hps[1], stream=B)
    st.sync()
    torch.cuda.synchronize()
    host = st.host.numpy().copy()
    sc = [oracle.adam_scalars(1e-3, 0.9, 0.999, 1e-8, 0.0, t) for t in (1, 2)]
    for c in range(st.n_chunks):
        lo, hi = c * chunk, c * chunk + st.chunk_len(c)
        acc = [oracle.offload_accumulate([contrib[s][mb][c] for mb in range(n_micro)], w) for s in (0, 1)]
        on_host = n_micro - 1 if fuse_last_2 else n_micro
        assert_grad_exact(host[lo:hi], oracle.offload_accumulate([contrib[1][mb][c] for mb in range(on_host)], w),
                          f"host chunk {c}")
        p1, m1, v1, _ = oracle.adam_step(p0[lo:hi], m0[lo:hi], v0[lo:hi], acc[0], sc[0])
        ref = oracle.adam_step(p1, m1, v1, acc[1], sc[1])
        assert_state_close(f32_to_host(st.master[lo:hi]), f32_to_host(st.exp_avg[lo:hi]),
                           f32_to_host(st.exp_avg_sq[lo:hi]), bf16_to_host(st.bf16[lo:hi]), ref,
                           f"chunk {c}")
    st.engine.close()
