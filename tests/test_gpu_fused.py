"""GPU parity of the fused reduce-scatter + owner update (zero_reduce_scatter_adam):
against the oracle element by element on ragged and multi-tile sizes and all
specialised rank counts, and bit-identical to the two separate calls at the
full size of the 7B-class layer and of an owner-share bucket."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as S
from gpu_helpers import assert_grad_exact, assert_state_close, bf16_to_dev, bf16_to_host, f32_to_dev, f32_to_host

pytestmark = pytest.mark.gpu

import zero_sharded_optimizer_reduce_amd as z  # noqa: E402  (a broken package must fail, not skip)


def _sc(hp):
    return oracle.adam_scalars(hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"], hp["step"])


def _hp(wd, t):
    return dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=wd, step=t)


@pytest.mark.parametrize("n_ranks", [1, 2, 3, 4, 8, 16])
@pytest.mark.parametrize("per_shard,write_grad", [(4, True), (1024 * 3 + 4, False), (1 << 16, True), (37, True)])
@pytest.mark.parametrize("wd,t", [(0.0, 1), (0.1, 1000)])
def test_fused_matches_oracle(n_ranks, per_shard, write_grad, wd, t):
    n_shards = n_ranks
    numel = per_shard * n_shards
    grads = S.host_rank_grads(7000 + n_ranks + per_shard, n_ranks, numel, scales=np.linspace(0.5, 2, n_ranks))
    w = oracle.weights_from_counts(list(range(5, 5 + n_ranks)))
    p, m, v = S.host_state(7100 + per_shard, numel, 0.02, 1e-4 if t > 1 else 0, 1e-6 if t > 1 else 0)
    sl = [slice(k * per_shard, (k + 1) * per_shard) for k in range(n_shards)]
    P = [f32_to_dev(p[s]) for s in sl]
    M = [f32_to_dev(m[s]) for s in sl]
    V = [f32_to_dev(v[s]) for s in sl]
    B = [torch.empty(per_shard, dtype=torch.bfloat16, device="cuda") for _ in sl]
    G = [torch.empty(per_shard, dtype=torch.float32, device="cuda") for _ in sl] if write_grad else None
    hp = _hp(wd, t)
    z.zero_reduce_scatter_adam([bf16_to_dev(g) for g in grads], w, P, M, V, B, hp, grad_out=G)
    assert z.zero_last_path_vectorized() == (1 if per_shard % 4 == 0 else 0)
    sc = _sc(hp)
    for k, s in enumerate(sl):
        red = oracle.reduce_owner_shard(grads, w, n_shards, k)
        if write_grad:
            assert_grad_exact(f32_to_host(G[k]), red, f"owner {k}")
        ref = oracle.adam_step(p[s], m[s], v[s], red, sc)
        assert_state_close(f32_to_host(P[k]), f32_to_host(M[k]), f32_to_host(V[k]), bf16_to_host(B[k]), ref,
                           f"owner {k}")


def test_fused_validation():
    t = [torch.zeros(8, device="cuda") for _ in range(2)]
    b = [torch.zeros(8, dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    g = [torch.zeros(16, dtype=torch.bfloat16, device="cuda")]
    with pytest.raises(z.ZeroError):           # master aliases exp_avg
        z.zero_reduce_scatter_adam(g, [1.0], t, t, [x.clone() for x in t], b, _hp(0.0, 1))
    with pytest.raises(z.ZeroError):
        z.zero_reduce_scatter_adam(g, [1.0], t, [x.clone() for x in t], [x.clone() for x in t], b, _hp(0.0, 0))
    with pytest.raises(ValueError):
        z.zero_reduce_scatter_adam(g, [1.0], t[:1], t[:1], t[:1], b[:1], _hp(0.0, 1))


def _layer_setup(seed, n):
    from synthetic.workloads import LAYER_7B as wl
    from zero_sharded_optimizer_reduce_amd.drivers import ShardedStep
    st = ShardedStep(S.unit_numels(S.workloads.layer_7b_tensors()), n)
    gen = S.DeviceGen(seed)
    st.load_master(gen.normal_(torch.empty(st.psi_pad, device="cuda"), wl.master_sigma, 0))
    return st, gen, wl


def test_fused_equals_separate_calls_on_the_7b_layer():
    n = 4
    a, gen, wl = _layer_setup(11, n)
    b, _, _ = _layer_setup(11, n)
    grads = [torch.empty(a.psi_pad, dtype=torch.bfloat16, device="cuda") for _ in range(n)]
    tmp = torch.empty(a.psi_pad, dtype=torch.float32, device="cuda")
    w = z.zero_rank_weights(wl.extra["token_counts"], n)
    gb = [torch.empty(a.shard, dtype=torch.float32, device="cuda") for _ in range(n)]
    for t in (1, 2, 3):
        for r in range(n):
            gen.bf16_normal_(grads[r], wl.grad_sigma, t, r, tmp=tmp)
        hp = wl.hparams(step=t)
        a.step(grads, w, hp)
        z.zero_reduce_scatter_adam(grads, w, b.master, b.exp_avg, b.exp_avg_sq, b.bf16, hp, grad_out=gb)
        b.all_gather()
    torch.cuda.synchronize()
    for xa, xb in zip(a.master + a.exp_avg + a.exp_avg_sq + a.grad, b.master + b.exp_avg + b.exp_avg_sq + gb):
        assert torch.equal(xa.view(torch.int32), xb.view(torch.int32))
    assert torch.equal(a.view.view(torch.int16), b.view.view(torch.int16))


@pytest.mark.parametrize("in_place", [False, True])
def test_fused_with_accumulator(in_place):
    # the last micro-batch of an accumulation: grad = acc + red, then update;
    # equal to the reduce kernel's accumulate mode followed by the update
    n, per_shard = 4, 4096 + 4
    numel = n * per_shard
    grads = S.host_rank_grads(7300, n, numel)
    w = oracle.weights_mean(n)
    rng = np.random.default_rng(7301)
    acc = [S.normal_f32(rng, per_shard, 3e-3) for _ in range(n)]
    p, m, v = S.host_state(7302, numel, 0.02, 1e-4, 1e-6)
    sl = [slice(k * per_shard, (k + 1) * per_shard) for k in range(n)]
    P = [f32_to_dev(p[s]) for s in sl]
    M = [f32_to_dev(m[s]) for s in sl]
    V = [f32_to_dev(v[s]) for s in sl]
    B = [torch.empty(per_shard, dtype=torch.bfloat16, device="cuda") for _ in sl]
    A = [f32_to_dev(a) for a in acc]
    G = A if in_place else [torch.empty(per_shard, dtype=torch.float32, device="cuda") for _ in sl]
    hp = _hp(0.1, 7)
    z.zero_reduce_scatter_adam([bf16_to_dev(g) for g in grads], w, P, M, V, B, hp, grad_out=G, grad_acc=A)
    sc = _sc(hp)
    for k, s in enumerate(sl):
        tot = acc[k] + oracle.reduce_owner_shard(grads, w, n, k)
        assert_grad_exact(f32_to_host(G[k]), tot, f"owner {k}")
        ref = oracle.adam_step(p[s], m[s], v[s], tot, sc)
        assert_state_close(f32_to_host(P[k]), f32_to_host(M[k]), f32_to_host(V[k]), bf16_to_host(B[k]), ref,
                           f"owner {k}")


def test_chain_backward_fused_equals_separate():
    from zero_sharded_optimizer_reduce_amd.drivers import Zero3Chain
    units = [("emb", [("e", 4 * 256 * 7)]), ("layer", [("a", 5000), ("b", 3000)]), ("head", [("h", 4 * 256 * 3)])]
    n = 4
    gen = S.DeviceGen(123)
    chains = [Zero3Chain(units, n), Zero3Chain(units, n)]
    for ch in chains:
        for k in range(n):
            gen.normal_(ch.master[k], 0.02, 1, k)
            ch.bf16[k].copy_(ch.master[k])
    w = z.zero_rank_weights([3, 5, 2, 7], n)
    tmp = torch.empty(chains[0].max_pad, device="cuda")
    for t in (1, 2):
        hp = _hp(0.1, t)
        for u in reversed(range(len(units))):
            pad = chains[0].units[u][2]
            for ch in chains:
                for r, g in enumerate(ch.grads):
                    gen.bf16_normal_(g[:pad], 1e-3, 50 + t, u, r, tmp=tmp[:pad])
            chains[0].backward_unit(u, w, hp)
            chains[1].backward_unit_fused(u, w, hp)
    torch.cuda.synchronize()
    a, b = chains
    for xa, xb in zip(a.master + a.exp_avg + a.exp_avg_sq, b.master + b.exp_avg + b.exp_avg_sq):
        assert torch.equal(xa.view(torch.int32), xb.view(torch.int32))
    for xa, xb in zip(a.bf16, b.bf16):
        assert torch.equal(xa.view(torch.int16), xb.view(torch.int16))


@pytest.mark.parametrize("fused", [False, True])
def test_chain_backward_regather(fused):
    # backward gathers each unit again before its reduce (essay, ZeRO-3 的一次完整计算):
    # the regathered view equals that step's forward view, and the state
    # equals the chain without the regather, bit for bit
    from zero_sharded_optimizer_reduce_amd.drivers import Zero3Chain
    units = [("emb", [("e", 4 * 256 * 5)]), ("layer", [("a", 4000), ("b", 1000)]), ("head", [("h", 4 * 256 * 2)])]
    n = 4
    gen = S.DeviceGen(321)
    chains = [Zero3Chain(units, n), Zero3Chain(units, n)]
    for ch in chains:
        for k in range(n):
            gen.normal_(ch.master[k], 0.02, 1, k)
            ch.bf16[k].copy_(ch.master[k])
    w = z.zero_rank_weights(None, n)
    tmp = torch.empty(chains[0].max_pad, device="cuda")
    for t in (1, 2):
        hp = _hp(0.0, t)
        fwd = {}
        for u in range(len(units)):
            for ch in chains:
                v = ch.forward_unit(u)
            fwd[u] = v.clone()
        for u in reversed(range(len(units))):
            pad = chains[0].units[u][2]
            for ch in chains:
                for r, g in enumerate(ch.grads):
                    gen.bf16_normal_(g[:pad], 1e-3, 70 + t, u, r, tmp=tmp[:pad])
            step = (lambda ch, **kw: ch.backward_unit_fused(u, w, hp, **kw)) if fused else \
                (lambda ch, **kw: ch.backward_unit(u, w, hp, **kw))
            step(chains[0])
            step(chains[1], regather=True)
            # the regathered view was written before this unit's update
            assert torch.equal(chains[1].view[:pad].view(torch.int16), fwd[u].view(torch.int16)), (t, u)
    torch.cuda.synchronize()
    a, b = chains
    for xa, xb in zip(a.master + a.exp_avg + a.exp_avg_sq, b.master + b.exp_avg + b.exp_avg_sq):
        assert torch.equal(xa.view(torch.int32), xb.view(torch.int32))
    for xa, xb in zip(a.bf16, b.bf16):
        assert torch.equal(xa.view(torch.int16), xb.view(torch.int16))
