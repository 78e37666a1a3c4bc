"""GPU parity past 32-bit element and byte counts: an owner update over
2^31 + 4100 elements, a reduce of four 2^31 + 1024-element contributions into
one shard, an all-gather of two shards of 2^32 + 64 bytes each, the fused
reduce + update over 2^31 + 4100 elements, and the gradient norm over
2^31 + 4100 elements (an input whose sum of squares is exact in FP64).  Checked
against the oracle on windows at the start, across the 2^31-element (and
2^32-byte) boundaries and at the ragged tail.  Each case allocates up to about
40 GB of HBM and frees it before the next."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as S
from gpu_helpers import assert_grad_exact, assert_state_close, bf16_to_host, f32_to_host

pytestmark = pytest.mark.gpu

import zero_sharded_optimizer_reduce_amd as z  # noqa: E402  (a broken package must fail, not skip)

W = 4096


def _windows(n):
    b = 1 << 31
    return sorted({0, b - W // 2, b - W, b, n - W, (n // 2) & ~3})


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_update_beyond_2_to_31_elements():
    n = (1 << 31) + 4100
    gen = S.DeviceGen(901)
    p = gen.normal_(torch.empty(n, device="cuda"), 0.02, 0)
    m = gen.normal_(torch.empty(n, device="cuda"), 1e-4, 1)
    v = gen.normal_(torch.empty(n, device="cuda"), 1e-6, 2).abs_()
    g = gen.normal_(torch.empty(n, device="cuda"), 1e-3, 3)
    b = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1, step=7)
    wins = _windows(n)
    before = {a: [f32_to_host(x[a:a + W]) for x in (p, m, v, g)] for a in wins}
    print(f"update n={n}", flush=True)
    z.zero_adam_shard_step(p, m, v, b, g, hp)
    assert z.zero_last_path_vectorized() == 1
    torch.cuda.synchronize()
    sc = oracle.adam_scalars(hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"], hp["step"])
    for a in wins:
        ref = oracle.adam_step(*before[a], sc)
        assert_state_close(f32_to_host(p[a:a + W]), f32_to_host(m[a:a + W]), f32_to_host(v[a:a + W]),
                           bf16_to_host(b[a:a + W]), ref, f"window {a}")
    del p, m, v, g, b
    _free()


def test_reduce_beyond_2_to_31_elements():
    n = (1 << 31) + 1024
    gen = S.DeviceGen(902)
    tmp = torch.empty(1 << 28, device="cuda")
    grads = []
    for r in range(4):
        x = torch.empty(n, dtype=torch.bfloat16, device="cuda")
        for lo in range(0, n, 1 << 28):
            hi = min(n, lo + (1 << 28))
            gen.bf16_normal_(x[lo:hi], 1e-3, r, lo >> 28, tmp=tmp[:hi - lo])
        grads.append(x)
    del tmp
    out = torch.empty(n, device="cuda")
    w = z.zero_rank_weights([4096, 3072, 4096, 2048], 4)
    print(f"reduce n={n}", flush=True)
    z.zero_reduce_scatter(grads, w, [out])
    assert z.zero_last_path_vectorized() == 1
    torch.cuda.synchronize()
    for a in _windows(n):
        ref = oracle.reduce_full([bf16_to_host(x[a:a + W]) for x in grads], w)
        assert_grad_exact(f32_to_host(out[a:a + W]), ref, f"window {a}")
    del grads, out
    _free()


def test_all_gather_beyond_2_to_32_bytes():
    shard_bytes = (1 << 32) + 64
    shards = [torch.empty(shard_bytes, dtype=torch.uint8, device="cuda") for _ in range(2)]
    for k, s in enumerate(shards):
        s.view(torch.int32)[:].copy_(torch.arange(shard_bytes // 4, device="cuda", dtype=torch.int32) * 3 + k)
    view = torch.empty(2 * shard_bytes, dtype=torch.uint8, device="cuda")
    print(f"all-gather shard_bytes={shard_bytes}", flush=True)
    z.zero_all_gather_layer(shards, view)
    torch.cuda.synchronize()
    for k in range(2):
        for a in (0, (1 << 32) - 4096, shard_bytes - 4096):
            got = view[k * shard_bytes + a: k * shard_bytes + a + 4096].cpu().numpy()
            exp = shards[k][a:a + 4096].cpu().numpy()
            assert np.array_equal(got, exp), (k, a)
            assert np.array_equal(exp.view(np.int32), (np.arange(a // 4, a // 4 + 1024, dtype=np.int64) * 3 + k)
                                  .astype(np.int32)), (k, a)
    del shards, view
    _free()


def test_fused_beyond_2_to_31_elements():
    n = (1 << 31) + 4100
    gen = S.DeviceGen(903)
    tmp = torch.empty(1 << 28, device="cuda")
    grads = []
    for r in range(4):
        x = torch.empty(n, dtype=torch.bfloat16, device="cuda")
        for lo in range(0, n, 1 << 28):
            hi = min(n, lo + (1 << 28))
            gen.bf16_normal_(x[lo:hi], 1e-3, r, lo >> 28, tmp=tmp[:hi - lo])
        grads.append(x)
    del tmp
    p = gen.normal_(torch.empty(n, device="cuda"), 0.02, 10)
    m = torch.zeros(n, device="cuda")
    v = torch.zeros(n, device="cuda")
    b = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    w = z.zero_rank_weights(None, 4)
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, step=1)
    wins = _windows(n)
    p0 = {a: f32_to_host(p[a:a + W]) for a in wins}
    print(f"fused n={n}", flush=True)
    z.zero_reduce_scatter_adam(grads, w, [p], [m], [v], [b], hp)
    assert z.zero_last_path_vectorized() == 1
    torch.cuda.synchronize()
    sc = oracle.adam_scalars(hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"], hp["step"])
    for a in wins:
        red = oracle.reduce_full([bf16_to_host(x[a:a + W]) for x in grads], w)
        z0 = np.zeros(W, np.float32)
        ref = oracle.adam_step(p0[a], z0, z0.copy(), red, sc)
        assert_state_close(f32_to_host(p[a:a + W]), f32_to_host(m[a:a + W]), f32_to_host(v[a:a + W]),
                           bf16_to_host(b[a:a + W]), ref, f"window {a}")
    del grads, p, m, v, b
    _free()


def test_norm_beyond_2_to_31_elements():
    # x_i = (i mod 3 + 1) * 2^-10: every square and every partial sum is exact in
    # FP64, so the sum of squares is exactly (c1 + 4 c2 + 9 c3) * 2^-20
    from zero_sharded_optimizer_reduce_amd import _lib
    n = (1 << 31) + 4100
    x = (torch.arange(n, device="cuda", dtype=torch.int64) % 3 + 1).to(torch.float32).mul_(2.0 ** -10)
    ws = torch.empty(_lib.ZERO_NORM_BLOCKS, dtype=torch.float64, device="cuda")
    out = torch.empty(1, dtype=torch.float64, device="cuda")
    print(f"norm n={n}", flush=True)
    z.zero_grad_norm_sq([x], ws, out)
    torch.cuda.synchronize()
    c = [(n + 2 - k) // 3 for k in range(3)]          # counts of i mod 3 == 0, 1, 2
    exact = (c[0] * 1 + c[1] * 4 + c[2] * 9) * 2.0 ** -20
    assert out.item() == exact, (out.item(), exact)
    del x, ws, out
    _free()
