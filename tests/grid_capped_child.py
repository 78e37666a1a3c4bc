"""Child process of test_gpu_grid_capped.py: with ZERO_BLOCKS_PER_CU set in
its environment (read once, at the library's first launch), every streaming
kernel runs on a grid capped at that many workgroups per compute unit, so
each workgroup loops over several tiles (the grid-stride form that arrays
beyond the uncapped grid also take).  Checks each call against the oracle
and exits 0, or raises."""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)
sys.path.insert(0, os.path.dirname(HERE))

import numpy as np  # noqa: E402
import torch  # noqa: E402

import oracle  # noqa: E402
import synthetic as S  # noqa: E402
from gpu_helpers import (assert_grad_exact, assert_state_close, bf16_to_dev, bf16_to_host, f32_to_dev,  # noqa: E402
                         f32_to_host)
import zero_sharded_optimizer_reduce_amd as z  # noqa: E402

assert os.environ.get("ZERO_BLOCKS_PER_CU"), "run with ZERO_BLOCKS_PER_CU set"
g = S.rng(7)
HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1, step=3)
SC = oracle.adam_scalars(1e-3, 0.9, 0.999, 1e-8, 0.1, 3)


def say(msg):
    print(f"grid-capped ({os.environ['ZERO_BLOCKS_PER_CU']} per CU): {msg}", flush=True)


def reduce_scatter(n_ranks, n_shards, per_shard, accumulate):
    numel = n_shards * per_shard
    grads = [S.bf16_normal(g, numel, 1e-3) for _ in range(n_ranks)]
    w = oracle.weights_from_counts(list(range(3, 3 + n_ranks)))
    acc = [(g.standard_normal(per_shard) * 1e-3).astype(np.float32) for _ in range(n_shards)]
    out = [f32_to_dev(a) for a in acc]
    z.zero_reduce_scatter([bf16_to_dev(x) for x in grads], w, out, accumulate=accumulate)
    vec = z.zero_last_path_vectorized()
    torch.cuda.synchronize()
    for k in range(n_shards):
        if accumulate:
            ref = oracle.reduce_accumulate(acc[k], [x[k * per_shard:(k + 1) * per_shard] for x in grads], w)
        else:
            ref = oracle.reduce_owner_shard(grads, w, n_shards, k)
        assert_grad_exact(f32_to_host(out[k]), ref, f"reduce shard {k}")
    say(f"reduce-scatter N={n_ranks} shards={n_shards} per_shard={per_shard} acc={accumulate} vec={vec}: exact")


def reduce_scatter_f32(n_ranks, n_shards, per_shard):
    numel = n_shards * per_shard
    grads = [(g.standard_normal(numel) * 1e-3).astype(np.float32) for _ in range(n_ranks)]
    w = oracle.weights_mean(n_ranks)
    out = [torch.empty(per_shard, dtype=torch.float32, device="cuda") for _ in range(n_shards)]
    z.zero_reduce_scatter_f32([f32_to_dev(x) for x in grads], w, out)
    torch.cuda.synchronize()
    for k in range(n_shards):
        assert_grad_exact(f32_to_host(out[k]), oracle.reduce_owner_shard(grads, w, n_shards, k), f"f32 shard {k}")
    say(f"reduce-scatter of FP32 contributions N={n_ranks} per_shard={per_shard} "
        f"vec={z.zero_last_path_vectorized()}: exact")


def adam(n, offset=0):
    """offset 1 puts every buffer one element past a 16-byte boundary: the
    element-wise kernel."""
    p, m, v = S.host_state(11, n, 0.02, 1e-4, 1e-6)
    gr = (g.standard_normal(n) * 1e-3).astype(np.float32)

    def dev(x):
        t = torch.zeros(n + offset, dtype=torch.float32, device="cuda")
        t[offset:].copy_(torch.from_numpy(x))
        return t[offset:]

    P, M, V, G = (dev(x) for x in (p, m, v, gr))
    B = torch.empty(n + offset, dtype=torch.bfloat16, device="cuda")[offset:]
    z.zero_adam_shard_step(P, M, V, B, G, HP)
    vec = z.zero_last_path_vectorized()
    torch.cuda.synchronize()
    u = assert_state_close(f32_to_host(P), f32_to_host(M), f32_to_host(V), bf16_to_host(B),
                           oracle.adam_step(p, m, v, gr, SC), f"adam n={n}")
    say(f"owner update n={n} vec={vec}: max ulp {u}")


def fused(n_ranks, n_shards, per_shard):
    numel = n_shards * per_shard
    grads = [S.bf16_normal(g, numel, 1e-3) for _ in range(n_ranks)]
    w = oracle.weights_mean(n_ranks)
    state = [S.host_state(20 + k, per_shard, 0.02, 1e-4, 1e-6) for k in range(n_shards)]
    acc = [(g.standard_normal(per_shard) * 1e-3).astype(np.float32) for _ in range(n_shards)]
    P = [f32_to_dev(s[0]) for s in state]
    M = [f32_to_dev(s[1]) for s in state]
    V = [f32_to_dev(s[2]) for s in state]
    B = [torch.empty(per_shard, dtype=torch.bfloat16, device="cuda") for _ in range(n_shards)]
    GA = [f32_to_dev(a) for a in acc]
    GO = [torch.empty(per_shard, dtype=torch.float32, device="cuda") for _ in range(n_shards)]
    z.zero_reduce_scatter_adam([bf16_to_dev(x) for x in grads], w, P, M, V, B, HP, grad_out=GO, grad_acc=GA)
    vec = z.zero_last_path_vectorized()
    torch.cuda.synchronize()
    for k in range(n_shards):
        red = oracle.reduce_accumulate(acc[k], [x[k * per_shard:(k + 1) * per_shard] for x in grads], w)
        assert_grad_exact(f32_to_host(GO[k]), red, f"fused gradient {k}")
        assert_state_close(f32_to_host(P[k]), f32_to_host(M[k]), f32_to_host(V[k]), bf16_to_host(B[k]),
                           oracle.adam_step(*state[k], red, SC), f"fused owner {k}")
    say(f"fused reduce + update N={n_ranks} shards={n_shards} per_shard={per_shard} vec={vec}: exact, ulp 0")


def gather(n_shards, shard_numel):
    shards = [S.bf16_normal(g, shard_numel, 1.0) for _ in range(n_shards)]
    view = torch.empty(n_shards * shard_numel, dtype=torch.bfloat16, device="cuda")
    z.zero_all_gather_layer([bf16_to_dev(x) for x in shards], view)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_to_host(view), oracle.all_gather(shards))
    say(f"all-gather shards={n_shards} shard={shard_numel}: exact")


torch.cuda.set_device(0)
reduce_scatter(4, 4, 600_004, False)
reduce_scatter(4, 4, 600_004, True)
reduce_scatter(3, 2, 400_000, False)
reduce_scatter(4, 3, 100_001, False)            # element-wise path
reduce_scatter_f32(4, 4, 300_000)
reduce_scatter_f32(4, 3, 100_001)              # element-wise path
adam(1_000_003)                                # vector path with a 3-element tail
adam(999_999, offset=1)                        # element-wise path
fused(4, 4, 500_000)
fused(5, 2, 300_000)
fused(4, 3, 100_001)                           # element-wise path
gather(4, 1_000_000)                           # 16-byte path
gather(3, 333_334)                             # 4-byte path
gather(3, 333_335)                             # byte path
say("all kernels match the oracle")
