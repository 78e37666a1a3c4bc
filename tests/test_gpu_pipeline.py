"""Gradient sharding under a micro-batched (pipeline) backward: the gradients
of each model chunk arrive once per micro-batch and are reduce-scattered as
they arrive, accumulating into the owners' shards (blog "数据并行与 ZeRO：三级分片
各省多少", section 和别的并行叠在一起: the gradient is reduced chunk by chunk
while it is being computed, not once at the end).  Checked against the oracle:
per chunk, the accumulated shard is r_1 + r_2 + ... in micro-batch order, then
the owners' update."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as S
from gpu_helpers import assert_grad_exact, assert_state_close, bf16_to_dev, bf16_to_host, f32_to_dev, f32_to_host

pytestmark = pytest.mark.gpu

import zero_sharded_optimizer_reduce_amd as z  # noqa: E402  (a broken package must fail, not skip)


def test_chunkwise_accumulating_reduce_scatter():
    n, M = 4, 3
    chunk_numels = [4 * 256 * 9, 4 * 256 * 3 + 1000, 4 * 256 * 17]   # model chunks, each its own layout
    layouts = [oracle.shard_layout([c], n) for c in chunk_numels]
    rng = np.random.default_rng(77)
    w = oracle.weights_from_counts([5, 3, 7, 1])
    # contributions[m][c][r]
    contrib = [[S.host_rank_grads(int(rng.integers(1 << 30)), n, pad) for (_, pad, _) in layouts]
               for _ in range(M)]
    gshards = [[torch.empty(s, dtype=torch.float32, device="cuda") for _ in range(n)] for (_, _, s) in layouts]
    for m in range(M):                          # micro-batches
        for c in reversed(range(len(layouts))):  # backward visits the chunks in reverse
            z.zero_reduce_scatter([bf16_to_dev(g) for g in contrib[m][c]], w, gshards[c], accumulate=m > 0)
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1, step=4)
    sc = oracle.adam_scalars(1e-3, 0.9, 0.999, 1e-8, 0.1, 4)
    for c, (psi, pad, s) in enumerate(layouts):
        p, mm, v = S.host_state(90 + c, pad, 0.02, 1e-4, 1e-6)
        for k in range(n):
            acc = None
            for m in range(M):
                r = oracle.reduce_owner_shard(contrib[m][c], w, n, k)
                acc = r if acc is None else acc + r
            assert_grad_exact(f32_to_host(gshards[c][k]), acc, f"chunk {c} owner {k}")
            sl = slice(k * s, (k + 1) * s)
            P, Mm, V = f32_to_dev(p[sl]), f32_to_dev(mm[sl]), f32_to_dev(v[sl])
            B = torch.empty(s, dtype=torch.bfloat16, device="cuda")
            z.zero_adam_shard_step(P, Mm, V, B, gshards[c][k], hp)
            ref = oracle.adam_step(p[sl], mm[sl], v[sl], acc, sc)
            assert_state_close(f32_to_host(P), f32_to_host(Mm), f32_to_host(V), bf16_to_host(B), ref,
                               f"chunk {c} owner {k}")
