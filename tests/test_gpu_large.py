"""GPU parity past 32-bit element and byte counts: an owner update over
2^31 + 4100 elements, a reduce of four 2^31 + 1024-element contributions into
one shard, and an all-gather of two shards of 2^32 + 64 bytes each.  Checked
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

z = pytest.importorskip("zero_sharded_optimizer_reduce_amd")

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
