"""The ZeRO-3 chain driver on a small model with ragged unit sizes, every
element against the oracle, for both backward forms the benchmark times:
the separate reduce-scatter and owner updates, and the fused reduce + update
(one launch per owner, the reduced shards never stored); with and without
gathering each unit again before its backward reduce (essay "把训练账本放进
多张设备", section ZeRO-3 的一次完整计算: the backward pass needs the layer's
weights again).  Two steps, so the second starts from the first's state.

Per unit and step: the forward view equals the owners' BF16 shards in owner
order (and, after the first step, the BF16 of the oracle's masters); the
reduced gradient (separate form) is bit-exact; master, m, v and the BF16
shard are at ulp distance 0."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as S
from gpu_helpers import assert_grad_exact, assert_state_close, bf16_to_host, f32_to_host
from synthetic.workloads import Workload

pytestmark = pytest.mark.gpu

import zero_sharded_optimizer_reduce_amd as z  # noqa: E402  (a broken package must fail, not skip)
from zero_sharded_optimizer_reduce_amd.drivers import Zero3Chain  # noqa: E402

# embedding-like, two ragged "layers" (padding to N*256 needed) and a head
UNITS = [("embedding", [("embedding", 3000 * 64)]),
         ("layer0", [("q", 64 * 64), ("k", 64 * 16), ("v", 64 * 16), ("o", 64 * 64), ("mlp", 3 * 64 * 170 + 7)]),
         ("layer1", [("q", 64 * 64), ("k", 64 * 16), ("v", 64 * 16), ("o", 64 * 64), ("mlp", 3 * 64 * 170 + 7)]),
         ("lm_head", [("lm_head", 3000 * 64)])]
WL = Workload(name="chain_small", description="small chain", psi=0, seed=31, weight_decay=0.1)


def _sc(hp):
    return oracle.adam_scalars(hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"], hp["step"])


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("regather", [False, True])
def test_small_chain_two_steps(fused, regather):
    n = 4
    ch = Zero3Chain(UNITS, n, device="cuda")
    U = len(ch.units)
    print(f"small chain fused={fused} regather={regather} units={[u[1:] for u in ch.units]}", flush=True)
    assert any(u[1] != u[2] for u in ch.units)            # some unit is padded
    gen = S.DeviceGen(WL.seed)
    for k in range(n):
        gen.normal_(ch.master[k], WL.master_sigma, 1, k)
        ch.bf16[k].copy_(ch.master[k])
        for x in (ch.exp_avg, ch.exp_avg_sq):
            x[k].zero_()
    torch.cuda.synchronize()

    def flat(bufs, u, host=f32_to_host):
        s, off = ch.units[u][3], ch.offsets[u]
        return np.concatenate([host(b[off:off + s]) for b in bufs])

    ref = {u: [flat(ch.master, u), np.zeros(ch.units[u][2], np.float32), np.zeros(ch.units[u][2], np.float32),
               flat(ch.bf16, u, bf16_to_host)] for u in range(U)}
    w = z.zero_rank_weights([5, 3, 2, 6], n)
    wo = oracle.weights_from_counts([5, 3, 2, 6])
    for t in (1, 2):
        hp = WL.hparams(step=t)
        sc = _sc(hp)
        for u in range(U):                                 # forward
            view = ch.forward_unit(u)
            torch.cuda.synchronize()
            assert np.array_equal(bf16_to_host(view), ref[u][3]), (t, u)
        for u in reversed(range(U)):                       # backward
            pad = ch.units[u][2]
            for r in range(n):
                gen.bf16_normal_(ch.grads[r][:pad], WL.grad_sigma, 100 * t + u, r)
            if fused:
                ch.backward_unit_fused(u, w, hp, regather=regather)
            else:
                ch.backward_unit(u, w, hp, regather=regather)
            torch.cuda.synchronize()
            if regather:                                   # the view gathered again before the reduce
                assert np.array_equal(bf16_to_host(ch.view[:pad]), ref[u][3]), (t, u)
            g = [bf16_to_host(x[:pad]) for x in ch.grads]
            red = oracle.reduce_full(g, wo)
            if not fused:
                s = ch.units[u][3]
                assert_grad_exact(np.concatenate([f32_to_host(x[:s]) for x in ch.grad_shards]), red,
                                  f"step {t} unit {u}")
            new = oracle.adam_step(ref[u][0], ref[u][1], ref[u][2], red, sc)
            assert_state_close(flat(ch.master, u), flat(ch.exp_avg, u), flat(ch.exp_avg_sq, u),
                               flat(ch.bf16, u, bf16_to_host), new, f"step {t} unit {u}")
            ref[u] = list(new)
