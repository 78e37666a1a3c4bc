"""GPU parity of each C-ABI call against the oracle, on sizes that span many
workgroup tiles plus ragged tails, every rank count the kernels specialise,
both the 16-byte and the element-wise paths, and the edge cases (empty input,
one rank, non-finite and subnormal values, BF16 rounding ties)."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as S
from gpu_helpers import (assert_grad_exact, assert_state_close, bf16_to_dev, bf16_to_host, f32_to_dev,
                         f32_to_host)

pytestmark = pytest.mark.gpu

import zero_sharded_optimizer_reduce_amd as z  # noqa: E402  (a broken package must fail, not skip)


def _sc(hp):
    return oracle.adam_scalars(hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"], hp["step"])


HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, step=1)


# ------------------------------------------------------------ reduce-scatter
@pytest.mark.parametrize("n_ranks", [1, 2, 3, 4, 5, 8, 16])
@pytest.mark.parametrize("per_shard", [8, 2048, 8 * 1000 + 8, 1 << 17])
def test_reduce_scatter_vector_path(n_ranks, per_shard):
    n_shards = n_ranks
    numel = per_shard * n_shards
    print(f"reduce_scatter n_ranks={n_ranks} numel={numel}", flush=True)
    grads = S.host_rank_grads(1000 + n_ranks, n_ranks, numel, scales=np.linspace(0.5, 2, n_ranks))
    w = oracle.weights_from_counts(list(range(7, 7 + n_ranks)))
    g_dev = [bf16_to_dev(g) for g in grads]
    out = [torch.empty(per_shard, dtype=torch.float32, device="cuda") for _ in range(n_shards)]
    z.zero_reduce_scatter(g_dev, w, out)
    assert z.zero_last_path_vectorized() == 1
    ref = oracle.reduce_scatter(grads, w, n_shards)
    for k in range(n_shards):
        assert_grad_exact(f32_to_host(out[k]), ref[k], f"shard {k}")
    # accumulate mode adds a second reduction on top
    grads2 = S.host_rank_grads(2000 + n_ranks, n_ranks, numel)
    z.zero_reduce_scatter([bf16_to_dev(g) for g in grads2], w, out, accumulate=True)
    for k in range(n_shards):
        ref2 = ref[k] + oracle.reduce_owner_shard(grads2, w, n_shards, k)
        assert_grad_exact(f32_to_host(out[k]), ref2, f"accumulated shard {k}")


@pytest.mark.parametrize("n_ranks,n_shards,numel", [(4, 4, 4 * 257), (3, 3, 3 * 5), (4, 1, 1001),
                                                      (1, 1, 1), (16, 16, 16 * 9), (2, 2, 2 * 4099)])
def test_reduce_scatter_element_path(n_ranks, n_shards, numel):
    grads = S.host_rank_grads(3000 + numel, n_ranks, numel)
    w = oracle.weights_from_counts(list(range(1, 1 + n_ranks)))
    out = [torch.empty(numel // n_shards, dtype=torch.float32, device="cuda") for _ in range(n_shards)]
    z.zero_reduce_scatter([bf16_to_dev(g) for g in grads], w, out)
    assert z.zero_last_path_vectorized() == 0
    for k, r in enumerate(oracle.reduce_scatter(grads, w, n_shards)):
        assert_grad_exact(f32_to_host(out[k]), r, f"shard {k}")


def test_reduce_scatter_misaligned_views_take_element_path():
    n, numel = 4, 4 * 1024
    grads = S.host_rank_grads(77, n, numel + 1)
    w = oracle.weights_mean(n)
    # views that start one BF16 element in: 2-byte aligned, not 16-byte aligned
    g_dev = [bf16_to_dev(g)[1:] for g in grads]
    out = [torch.empty(numel // n, dtype=torch.float32, device="cuda") for _ in range(n)]
    z.zero_reduce_scatter(g_dev, w, out)
    assert z.zero_last_path_vectorized() == 0
    for k, r in enumerate(oracle.reduce_scatter([g[1:] for g in grads], w, n)):
        assert_grad_exact(f32_to_host(out[k]), r)


def test_reduce_scatter_empty_and_errors():
    out = [torch.empty(0, dtype=torch.float32, device="cuda") for _ in range(4)]
    z.zero_reduce_scatter([torch.empty(0, dtype=torch.bfloat16, device="cuda")] * 4, [0.25] * 4, out)
    g = [torch.zeros(16, dtype=torch.bfloat16, device="cuda") for _ in range(4)]
    with pytest.raises(ValueError):
        z.zero_reduce_scatter(g, [0.25] * 4, [torch.empty(5, device="cuda") for _ in range(3)])
    # output overlapping an input is rejected by the library before any launch
    buf = torch.zeros(64, dtype=torch.float32, device="cuda")
    gb = buf.view(torch.bfloat16)[:64]
    with pytest.raises(z.ZeroError):
        z.zero_reduce_scatter([gb], [1.0], [buf[:64]])


def test_reduce_special_values():
    vals = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 1e-40, -1e-40, 3e38, -3e38, 1.0, 2 ** -133],
                    np.float32)
    n = 4
    rng = np.random.default_rng(5)
    numel = 8 * 64
    grads = [S.to_bf16_bits(rng.choice(vals, numel).astype(np.float32)) for _ in range(n)]
    w = np.array([0.5, 0.25, 0.125, 0.125], np.float32)
    out = [torch.empty(numel, dtype=torch.float32, device="cuda")]
    z.zero_reduce_scatter([bf16_to_dev(g) for g in grads], w, out)
    assert_grad_exact(f32_to_host(out[0]), oracle.reduce_full(grads, w))


# --------------------------------------------------------------------- Adam
@pytest.mark.parametrize("n", [0, 1, 3, 4, 5, 1023, 4096 + 3, 257 * 1024 + 1])
@pytest.mark.parametrize("wd,step", [(0.0, 1), (0.1, 2), (0.1, 1000)])
def test_adam_vector_path(n, wd, step):
    print(f"adam n={n} wd={wd} step={step}", flush=True)
    p, m, v = S.host_state(4000 + n, n, 0.02, 1e-4 if step > 1 else 0.0, 1e-6 if step > 1 else 0.0)
    g = S.normal_f32(S.rng(5000 + n), n, 1e-3)
    hp = dict(HP, weight_decay=wd, step=step)
    P, M, V, G = (f32_to_dev(x) for x in (p, m, v, g))
    B = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    z.zero_adam_shard_step(P, M, V, B, G, hp)
    ref = oracle.adam_step(p, m, v, g, _sc(hp))
    u = assert_state_close(f32_to_host(P), f32_to_host(M), f32_to_host(V), bf16_to_host(B), ref)
    print(f"  max ulps {u}", flush=True)


@pytest.mark.parametrize("n", [1, 7, 1000, 4099])
def test_adam_element_path(n):
    p, m, v = S.host_state(6000 + n, n + 1, 0.02, 1e-4, 1e-6)
    g = S.normal_f32(S.rng(6100 + n), n + 1, 1e-3)
    hp = dict(HP, weight_decay=0.1, step=10)
    P, M, V, G = (f32_to_dev(x)[1:] for x in (p, m, v, g))      # 4-byte, not 16-byte aligned
    B = torch.empty(n + 1, dtype=torch.bfloat16, device="cuda")[1:]
    z.zero_adam_shard_step(P, M, V, B, G, hp)
    assert z.zero_last_path_vectorized() == 0
    ref = oracle.adam_step(p[1:], m[1:], v[1:], g[1:], _sc(hp))
    assert_state_close(f32_to_host(P), f32_to_host(M), f32_to_host(V), bf16_to_host(B), ref)


def test_adam_special_values_and_ties():
    specials = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 1e-40, -1e-40, 1e-45, 3e38, -3e38,
                         1e-20, 1e20], np.float32)
    rng = np.random.default_rng(11)
    n = 4096
    p = rng.choice(specials, n).astype(np.float32)
    # masters exactly halfway between two bf16 values, both parities, and
    # values one ulp either side of a tie
    ties = (rng.integers(0x3C000000, 0x3F800000, n, dtype=np.uint32) & 0xFFFF0000) | 0x8000
    p[: n // 2] = ties[: n // 2].view(np.float32)
    p[n // 2: n // 2 + 256] = (ties[:256] + 1).view(np.float32)
    m = rng.choice(specials, n).astype(np.float32)
    v = np.abs(rng.choice(specials, n)).astype(np.float32)
    g = rng.choice(specials, n).astype(np.float32)
    g[: n // 2] = 0.0                       # with wd=0 the tie masters pass through unchanged
    m[: n // 2] = 0.0
    v[: n // 2] = 0.0
    for wd in (0.0, 0.1):
        hp = dict(HP, weight_decay=wd, step=3)
        P, M, V, G = (f32_to_dev(x) for x in (p, m, v, g))
        B = torch.empty(n, dtype=torch.bfloat16, device="cuda")
        z.zero_adam_shard_step(P, M, V, B, G, hp)
        ref = oracle.adam_step(p, m, v, g, _sc(hp))
        assert_state_close(f32_to_host(P), f32_to_host(M), f32_to_host(V), bf16_to_host(B), ref, f"wd={wd}")


def test_adam_rejects_bad_hparams():
    t = torch.zeros(8, device="cuda")
    b = torch.zeros(8, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(z.ZeroError):
        z.zero_adam_shard_step(t, t.clone(), t.clone(), b, t.clone(), dict(HP, step=0))
    with pytest.raises(z.ZeroError):      # master aliasing grad
        z.zero_adam_shard_step(t, t.clone(), t.clone(), b, t, HP)


def test_adam_scalars_match_oracle():
    for step in (1, 2, 3, 10, 1000, 123456):
        for wd in (0.0, 0.1):
            hp = dict(HP, step=step, weight_decay=wd)
            lib = z.zero_adam_scalars_compute(hp)
            ref = _sc(hp)
            for k in ref:
                assert lib[k].view(np.uint32) == ref[k].view(np.uint32), (k, step)


# --------------------------------------------------------------- all-gather
@pytest.mark.parametrize("dtype,shard_elems", [(torch.bfloat16, 1 << 16), (torch.bfloat16, 1000 * 8 + 2),
                                               (torch.float32, 12345), (torch.uint8, 1001),
                                               (torch.bfloat16, 1)])
@pytest.mark.parametrize("n_shards", [1, 3, 4, 16])
def test_all_gather(dtype, shard_elems, n_shards):
    torch.manual_seed(shard_elems + n_shards)
    if dtype == torch.uint8:
        shards = [torch.randint(0, 255, (shard_elems,), dtype=dtype, device="cuda") for _ in range(n_shards)]
    else:
        shards = [torch.randn(shard_elems, device="cuda").to(dtype) for _ in range(n_shards)]
    view = torch.empty(shard_elems * n_shards, dtype=dtype, device="cuda")
    z.zero_all_gather_layer(shards, view)
    got = view.view(torch.uint8).cpu().numpy()
    ref = oracle.all_gather([s.view(torch.uint8).cpu().numpy() for s in shards])
    assert np.array_equal(got, ref)


# --------------------------------------------- FP32 contributions (gradients kept in FP32)
@pytest.mark.parametrize("n_ranks,per_shard", [(4, 4096 + 4), (3, 1024), (4, 37), (1, 8), (16, 64)])
@pytest.mark.parametrize("accumulate", [False, True])
def test_reduce_scatter_f32_contributions(n_ranks, per_shard, accumulate):
    n_shards = n_ranks
    numel = per_shard * n_shards
    rng = np.random.default_rng(8000 + per_shard + n_ranks)
    grads = [S.normal_f32(rng, numel, 1e-3) for _ in range(n_ranks)]
    w = oracle.weights_from_counts(list(range(2, 2 + n_ranks)))
    init = [S.normal_f32(rng, per_shard, 1e-3) for _ in range(n_shards)]
    out = [f32_to_dev(x) for x in init]
    z.zero_reduce_scatter_f32([f32_to_dev(g) for g in grads], w, out, accumulate=accumulate)
    assert z.zero_last_path_vectorized() == (1 if per_shard % 4 == 0 else 0)
    for k in range(n_shards):
        red = oracle.reduce_owner_shard(grads, w, n_shards, k)
        ref = init[k] + red if accumulate else red
        assert_grad_exact(f32_to_host(out[k]), ref, f"shard {k}")
