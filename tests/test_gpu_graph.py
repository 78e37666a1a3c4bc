"""GPU parity of the graph-capturable forms (the Adam scalars read from device
memory when the kernels run):

* zero_adam_shard_step_dev equals zero_adam_shard_step bit for bit, with and
  without decay (decided in the kernel from the device value), on the vector
  and element paths, with special values, with and without a gradient scale;
* zero_reduce_scatter_adam_dev equals zero_reduce_scatter_adam;
* a ShardedStep captured into a HIP graph and replayed over several steps
  (new contributions and new step counts each time, eager work and
  synchronisations between replays) equals the eager step after every replay;
* the same with the host queueing every step before the device runs the
  first (ring slots reused under the completion events only);
* zero_adam_scalars_fetch walks its ring slot by slot and sees slots the
  host rewrote between calls;
* invalid device-scalar and ring arguments are rejected before anything is
  launched.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic as S
from gpu_helpers import f32_to_dev

pytestmark = pytest.mark.gpu

import zero_sharded_optimizer_reduce_amd as z  # noqa: E402  (a broken package must fail, not skip)
from zero_sharded_optimizer_reduce_amd import _lib  # noqa: E402
from zero_sharded_optimizer_reduce_amd.drivers import GraphedStep, ShardedStep  # noqa: E402


def _hp(wd, t):
    return dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=wd, step=t)


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


def _same(a, b, what):
    assert torch.equal(_bits(a), _bits(b)), what


def _state(n, seed, special=False):
    rng = np.random.default_rng(seed)
    p = S.normal_f32(rng, n, 0.02)
    m = S.normal_f32(rng, n, 1e-4)
    v = np.abs(S.normal_f32(rng, n, 1e-6))
    g = S.normal_f32(rng, n, 1e-3)
    if special:
        sv = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 1e-40, -1e-40, 3e38], np.float32)
        p[:8], g[8:16], m[16:24] = sv, sv, sv
        p[24:32], g[24:32] = -0.0, -0.0
    return [f32_to_dev(x) for x in (p, m, v, g)]


@pytest.mark.parametrize("n,offset", [(4096 * 3 + 4, 0), (4096 + 3, 0), (4096 + 3, 1)])
@pytest.mark.parametrize("wd", [0.0, 0.1])
@pytest.mark.parametrize("scaled", [False, True])
def test_update_with_device_scalars_equals_host_scalars(n, offset, wd, scaled):
    # offset 1: views one element into their buffers, so the element-wise kernels run
    hp = _hp(wd, 5)
    a = [x[offset:] for x in _state(n + offset, 11, special=True)]
    b = [x.clone()[offset:] for x in _state(n + offset, 11, special=True)]
    ba = torch.empty(n + offset, dtype=torch.bfloat16, device="cuda")[offset:]
    bb = torch.empty(n + offset, dtype=torch.bfloat16, device="cuda")[offset:]
    scale = torch.tensor([0.37], device="cuda") if scaled else None
    if scaled:
        z.zero_adam_shard_step_scaled(a[0], a[1], a[2], ba, a[3], scale, hp)
    else:
        z.zero_adam_shard_step(a[0], a[1], a[2], ba, a[3], hp)
    dev = z.adam_scalars_tensor(hp).cuda()
    z.zero_adam_shard_step_dev(b[0], b[1], b[2], bb, b[3], dev, grad_scale=scale)
    assert z.zero_last_path_vectorized() == (0 if offset else 1)
    torch.cuda.synchronize()
    for x, y, name in zip(a[:3] + [ba], b[:3] + [bb], ("master", "exp_avg", "exp_avg_sq", "bf16")):
        _same(x, y, f"{name} n={n} wd={wd} scaled={scaled}")


@pytest.mark.parametrize("wd", [0.0, 0.1])
@pytest.mark.parametrize("with_acc", [False, True])
@pytest.mark.parametrize("per", [4096 + 4, 1001])
def test_fused_with_device_scalars_equals_host_scalars(wd, with_acc, per):
    n = 4
    grads = [S.bf16_normal(np.random.default_rng(r + 30), n * per, 1e-3) for r in range(n)]
    gd = [torch.from_numpy(g.view(np.int16)).cuda().view(torch.bfloat16) for g in grads]
    w = oracle.weights_from_counts([3, 5, 2, 7])
    hp = _hp(wd, 9)
    sets = []
    for _ in range(2):
        st = [_state(per, 40 + k) for k in range(n)]
        sets.append(dict(p=[s[0] for s in st], m=[s[1] for s in st], v=[s[2] for s in st],
                         b=[torch.empty(per, dtype=torch.bfloat16, device="cuda") for _ in range(n)],
                         g=[torch.empty(per, device="cuda") for _ in range(n)],
                         acc=[s[3] for s in st] if with_acc else None))
    A, B = sets
    z.zero_reduce_scatter_adam(gd, w, A["p"], A["m"], A["v"], A["b"], hp, grad_out=A["g"], grad_acc=A["acc"])
    z.zero_reduce_scatter_adam_dev(gd, w, B["p"], B["m"], B["v"], B["b"], z.adam_scalars_tensor(hp).cuda(),
                                   grad_out=B["g"], grad_acc=B["acc"])
    torch.cuda.synchronize()
    for key in ("p", "m", "v", "b", "g"):
        for k in range(n):
            _same(A[key][k], B[key][k], f"{key}[{k}]")


@pytest.mark.parametrize("fused", [False, True])
def test_graph_replays_equal_eager_steps(fused):
    numels = [4096 * 7, 1000, 4096 * 3 + 12]
    n = 4
    gen = S.DeviceGen(77)
    eager, graphed = ShardedStep(numels, n), ShardedStep(numels, n)
    master0 = gen.normal_(torch.empty(eager.psi_pad, device="cuda"), 0.02, 0)
    eager.load_master(master0)
    graphed.load_master(master0)
    w = z.zero_rank_weights([4096, 3072, 4096, 2048], n)
    grads = [torch.empty(eager.psi_pad, dtype=torch.bfloat16, device="cuda") for _ in range(n)]
    tmp = torch.empty(eager.psi_pad, device="cuda")
    g = GraphedStep(graphed, grads, w, fused=fused)
    for t in range(1, 2 * GraphedStep.RING + 4):   # every ring slot reused at least twice
        for r in range(n):
            gen.bf16_normal_(grads[r], 1e-3, t, r, tmp=tmp)
        hp = _hp(0.1 if t % 2 else 0.0, t)
        eager.step(grads, w, hp)
        g.step(hp)
        torch.cuda.synchronize()
        for name in ("master", "exp_avg", "exp_avg_sq", "bf16", "grad"):
            for k in range(n):
                _same(getattr(eager, name)[k], getattr(graphed, name)[k], f"step {t} {name}[{k}]")
        _same(eager.view, graphed.view, f"step {t} view")
        # unrelated eager work and a synchronisation before the next replay
        tmp.mul_(0.5).add_(1.0)
        torch.cuda.synchronize()


@pytest.mark.parametrize("fused", [False, True])
def test_graph_replays_without_host_waits(fused):
    # the host queues every step before the device has run the first one, so
    # ring slots are rewritten only as the completion events allow
    numels = [4096 * 5 + 8, 999]
    n = 4
    gen = S.DeviceGen(78)
    eager, graphed = ShardedStep(numels, n), ShardedStep(numels, n)
    master0 = gen.normal_(torch.empty(eager.psi_pad, device="cuda"), 0.02, 0)
    eager.load_master(master0)
    graphed.load_master(master0)
    w = z.zero_rank_weights([4096, 3072, 4096, 2048], n)
    grads = [gen.bf16_normal_(torch.empty(eager.psi_pad, dtype=torch.bfloat16, device="cuda"), 1e-3, 1, r)
             for r in range(n)]
    g = GraphedStep(graphed, grads, w, fused=fused)
    steps = 3 * GraphedStep.RING + 1
    hps = [_hp(0.1 if t % 3 else 0.0, t) for t in range(1, steps + 1)]
    for hp in hps:
        eager.step(grads, w, hp)
    for hp in hps:
        g.step(hp)
    torch.cuda.synchronize()
    for name in ("master", "exp_avg", "exp_avg_sq", "bf16", "grad"):
        for k in range(n):
            _same(getattr(eager, name)[k], getattr(graphed, name)[k], f"{name}[{k}] after {steps} steps")
    _same(eager.view, graphed.view, "view")


def test_scalars_fetch_walks_the_ring():
    R = 4
    F = z.ADAM_SCALARS_FLOATS
    ring = torch.zeros(R, F, dtype=torch.float32, pin_memory=True)
    for i in range(R):
        z.adam_scalars_tensor(_hp(0.1 * (i % 2), i + 1), out=ring[i])
    cursor = torch.zeros(1, dtype=torch.int32, device="cuda")
    dev = torch.zeros(F, device="cuda")
    for c in range(3 * R + 1):
        z.zero_adam_scalars_fetch(ring, cursor, dev)
        torch.cuda.synchronize()
        assert cursor.item() == c + 1
        _same(dev.cpu(), ring[c % R], f"call {c}")
        # rewrite the slot just read: the next pass over the ring must see the new values
        z.adam_scalars_tensor(_hp(0.1, 100 + c), out=ring[c % R])


def test_scalars_fetch_validation():
    lib = z.load()
    F = z.ADAM_SCALARS_FLOATS
    ring = torch.zeros(4, F, dtype=torch.float32, pin_memory=True)
    cursor = torch.zeros(2, dtype=torch.int32, device="cuda")
    dev = torch.zeros(F, device="cuda")
    rp, cp, dp = ring.data_ptr(), cursor.data_ptr(), dev.data_ptr()
    pageable = np.zeros(4 * F, np.float32)
    on_device = torch.zeros(4 * F, device="cuda")
    assert lib.zero_adam_scalars_fetch(rp, 3, cp, dp, None) == _lib.ZERO_ERR_ARG       # not a power of two
    assert lib.zero_adam_scalars_fetch(rp, 0, cp, dp, None) == _lib.ZERO_ERR_ARG
    assert lib.zero_adam_scalars_fetch(rp, 1 << 17, cp, dp, None) == _lib.ZERO_ERR_ARG
    assert lib.zero_adam_scalars_fetch(None, 4, cp, dp, None) == _lib.ZERO_ERR_ARG
    assert lib.zero_adam_scalars_fetch(rp, 4, None, dp, None) == _lib.ZERO_ERR_ARG
    assert lib.zero_adam_scalars_fetch(rp + 2, 4, cp, dp, None) == _lib.ZERO_ERR_ALIGN
    assert lib.zero_adam_scalars_fetch(rp, 4, dp, dp, None) == _lib.ZERO_ERR_ARG       # cursor inside scalars
    assert lib.zero_adam_scalars_fetch(pageable.ctypes.data, 4, cp, dp, None) == _lib.ZERO_ERR_ARG
    assert lib.zero_adam_scalars_fetch(on_device.data_ptr(), 4, cp, dp, None) == _lib.ZERO_ERR_ARG
    assert lib.zero_adam_scalars_fetch(rp, 1 << 16, cp, dp, None) == _lib.ZERO_ERR_ARG  # past the allocation
    with pytest.raises(ValueError):
        z.zero_adam_scalars_fetch(torch.zeros(4, F), cursor[:1], dev)                  # not pinned
    with pytest.raises(ValueError):
        z.zero_adam_scalars_fetch(torch.zeros(5, dtype=torch.float32, pin_memory=True), cursor[:1], dev)
    torch.cuda.synchronize()
    assert torch.count_nonzero(cursor) == 0 and torch.count_nonzero(dev) == 0           # nothing launched
    # a valid call after the rejected ones: no error was left behind
    z.adam_scalars_tensor(_hp(0.1, 7), out=ring[0])
    z.zero_adam_scalars_fetch(ring, cursor[:1], dev)
    torch.cuda.synchronize()
    assert cursor[0].item() == 1 and cursor[1].item() == 0
    _same(dev.cpu(), ring[0], "slot 0")


def test_device_scalar_arguments_are_validated():
    lib = z.load()
    n = 1024
    p, m, v, g = (torch.zeros(n, device="cuda") for _ in range(4))
    b = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    dev = z.adam_scalars_tensor(_hp(0.0, 1)).cuda()
    ptr = [t.data_ptr() for t in (p, m, v, b, g)]
    assert lib.zero_adam_shard_step_dev(*ptr, None, n, None, None) == _lib.ZERO_ERR_ARG
    assert lib.zero_adam_shard_step_dev(*ptr, None, n, dev.data_ptr() + 2, None) == _lib.ZERO_ERR_ALIGN
    with pytest.raises(z.ZeroError, match="ZERO_ERR_ARG"):      # the scalars inside an output
        z.zero_adam_shard_step_dev(p, m, v, b, g, m[100:100 + z.ADAM_SCALARS_FLOATS])
    with pytest.raises(ValueError):
        z.zero_adam_shard_step_dev(p, m, v, b, g, dev[:4])
    torch.cuda.synchronize()
    assert torch.count_nonzero(p) == 0 and torch.count_nonzero(m) == 0
    # the same scalars in the read-only gradient are allowed
    g[:z.ADAM_SCALARS_FLOATS] = dev
    z.zero_adam_shard_step_dev(p, m, v, b, g, g[:z.ADAM_SCALARS_FLOATS])
    torch.cuda.synchronize()


def test_graph_replays_equal_eager_steps_on_the_7b_layer():
    # the configuration the benchmark's graph variant times, at full size
    from synthetic.workloads import LAYER_7B as wl
    n = wl.n_ranks
    numels = S.unit_numels(S.workloads.layer_7b_tensors())
    gen = S.DeviceGen(wl.seed + 60)
    eager, graphed = ShardedStep(numels, n), ShardedStep(numels, n)
    master0 = gen.normal_(torch.empty(eager.psi_pad, device="cuda"), wl.master_sigma, 0)
    eager.load_master(master0)
    graphed.load_master(master0)
    del master0
    w = z.zero_rank_weights(wl.extra["token_counts"], n)
    grads = [torch.empty(eager.psi_pad, dtype=torch.bfloat16, device="cuda") for _ in range(n)]
    tmp = torch.empty(eager.psi_pad, device="cuda")
    g = GraphedStep(graphed, grads, w)
    for t in range(1, 4):
        print(f"7B layer graph replay, step {t}", flush=True)
        for r in range(n):
            gen.bf16_normal_(grads[r], wl.grad_sigma, t, r, tmp=tmp)
        hp = wl.hparams(step=t)
        eager.step(grads, w, hp)
        g.step(hp)
        torch.cuda.synchronize()
        for name in ("master", "exp_avg", "exp_avg_sq", "bf16", "grad"):
            for k in range(n):
                _same(getattr(eager, name)[k], getattr(graphed, name)[k], f"step {t} {name}[{k}]")
        _same(eager.view, graphed.view, f"step {t} view")
