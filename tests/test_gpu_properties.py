"""Randomised GPU parity: hypothesis draws combinations the fixed grids of the
other GPU tests do not enumerate (arbitrary float32 rank weights, any number
of ranks and owners up to 16, ragged shard lengths on both kernel paths,
accumulation, decay and step counts together) and every output is compared
with the oracle: reduced gradients bit for bit, master/m/v/BF16 at ulp
distance 0.  Derandomised, so every run checks the same cases."""
import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle
import synthetic as S
from gpu_helpers import assert_grad_exact, assert_state_close, bf16_to_dev, bf16_to_host, f32_to_dev, f32_to_host

pytestmark = pytest.mark.gpu

import zero_sharded_optimizer_reduce_amd as z  # noqa: E402  (a broken package must fail, not skip)

SETTINGS = settings(max_examples=30, deadline=None, derandomize=True, database=None,
                    suppress_health_check=list(HealthCheck))


def _weights(seed, n):
    """Arbitrary positive float32 weights (not normalised: the reduction takes
    whatever the caller passes)."""
    return (np.random.default_rng(seed).uniform(0.05, 1.5, n)).astype(np.float32)


def _sc(hp):
    return oracle.adam_scalars(hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"], hp["step"])


@SETTINGS
@given(n_ranks=st.integers(1, 16), n_shards=st.integers(1, 16), per_shard=st.integers(1, 3000),
       accumulate=st.booleans(), seed=st.integers(0, 10 ** 6))
def test_reduce_scatter_random_cases(n_ranks, n_shards, per_shard, accumulate, seed):
    numel = per_shard * n_shards
    grads = S.host_rank_grads(seed, n_ranks, numel, sigma=float(10.0 ** (seed % 7 - 5)))
    w = _weights(seed, n_ranks)
    acc0 = S.normal_f32(S.rng(seed + 1), numel, 1e-3)
    outs = [f32_to_dev(acc0[k * per_shard:(k + 1) * per_shard]) for k in range(n_shards)]
    z.zero_reduce_scatter([bf16_to_dev(g) for g in grads], w, outs, accumulate=accumulate)
    torch.cuda.synchronize()
    ref = oracle.reduce_accumulate(acc0, grads, w) if accumulate else oracle.reduce_full(grads, w)
    for k in range(n_shards):
        assert_grad_exact(f32_to_host(outs[k]), ref[k * per_shard:(k + 1) * per_shard],
                          f"owner {k} of {n_shards}, {n_ranks} ranks, {per_shard} per shard")


@SETTINGS
@given(n_ranks=st.integers(1, 16), n_shards=st.integers(1, 8), per_shard=st.integers(1, 3000),
       with_acc=st.booleans(), write_grad=st.booleans(), wd=st.sampled_from([0.0, 0.01, 0.1]),
       step=st.integers(1, 5000), seed=st.integers(0, 10 ** 6))
def test_fused_random_cases(n_ranks, n_shards, per_shard, with_acc, write_grad, wd, step, seed):
    numel = per_shard * n_shards
    grads = S.host_rank_grads(seed, n_ranks, numel)
    w = _weights(seed + 2, n_ranks)
    mid_run = step > 1
    p, m, v = S.host_state(seed + 3, numel, 0.02, 1e-4 if mid_run else 0.0, 1e-6 if mid_run else 0.0)
    acc0 = S.normal_f32(S.rng(seed + 4), numel, 1e-3)
    sl = [slice(k * per_shard, (k + 1) * per_shard) for k in range(n_shards)]
    P, M, V = ([f32_to_dev(x[s]) for s in sl] for x in (p, m, v))
    B = [torch.empty(per_shard, dtype=torch.bfloat16, device="cuda") for _ in sl]
    A = [f32_to_dev(acc0[s]) for s in sl] if with_acc else None
    G = [torch.empty(per_shard, dtype=torch.float32, device="cuda") for _ in sl] if write_grad else None
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=wd, step=step)
    z.zero_reduce_scatter_adam([bf16_to_dev(g) for g in grads], w, P, M, V, B, hp, grad_out=G, grad_acc=A)
    torch.cuda.synchronize()
    sc = _sc(hp)
    red = oracle.reduce_accumulate(acc0, grads, w) if with_acc else oracle.reduce_full(grads, w)
    for k, s in enumerate(sl):
        what = f"owner {k} of {n_shards}, {n_ranks} ranks, {per_shard} per shard, t={step}, wd={wd}"
        if write_grad:
            assert_grad_exact(f32_to_host(G[k]), red[s], what)
        ref = oracle.adam_step(p[s], m[s], v[s], red[s], sc)
        assert_state_close(f32_to_host(P[k]), f32_to_host(M[k]), f32_to_host(V[k]), bf16_to_host(B[k]), ref, what)
