"""Invariants the pages state, checked on the oracle (CPU only):

* sharded owners train the same model as replicated DP (slide, beat b3 and note
  原 N48; essay, section ZeRO-3 的一次完整计算);
* the next all-gather returns the one new version of the parameters;
* gradient buckets change nothing (essay, section ZeRO-3 的一次完整计算, the
  bucketing paragraph);
plus a scalar brute force of the vectorised code on tiny tensors.
"""
import struct

import numpy as np
import pytest

import oracle
import synthetic as S


def _sc(step=1, wd=0.0):
    return oracle.adam_scalars(1e-3, 0.9, 0.999, 1e-8, wd, step)


def _setup(n, psi, seed, counts=None):
    g = S.host_rank_grads(seed, n, psi, scales=np.linspace(0.5, 2.0, n))
    p, m, v = S.host_state(seed + 1, psi, 0.02, 1e-4, 1e-6)
    w = oracle.weights_mean(n) if counts is None else oracle.weights_from_counts(counts)
    return g, p, m, v, w


@pytest.mark.parametrize("n,wd,t", [(4, 0.0, 1), (4, 0.1, 3), (2, 0.1, 1000), (8, 0.0, 2), (3, 0.1, 5)])
def test_sharded_equals_replicated(n, wd, t):
    psi = n * 256 * 5
    g, p, m, v, w = _setup(n, psi, 40 + n, counts=list(range(3, 3 + n)))
    sc = _sc(t, wd)
    gd, pd, md, vd, bd = oracle.ddp_step(g, w, p, m, v, sc)
    sl = [oracle.shard_bounds(psi, n, k) for k in range(n)]
    outs, view = oracle.sharded_step(g, w, [p[a:b] for a, b in sl], [m[a:b] for a, b in sl],
                                     [v[a:b] for a, b in sl], sc)
    cat = lambda i: np.concatenate([o[i] for o in outs])
    for i, ref in enumerate((gd, pd, md, vd)):
        assert np.array_equal(cat(i).view(np.uint32), ref.view(np.uint32)), i
    assert np.array_equal(view, bd)
    # the gathered view is the single new version: bf16 of the new masters
    assert np.array_equal(view, oracle.f32_to_bf16_rne(cat(1)))


def test_buckets_equal_unbucketed():
    n, psi, bucket = 4, 10_000, 1536
    g, p, m, v, w = _setup(n, psi, 50)
    sc = _sc(1000, 0.1)
    g_full = oracle.reduce_full(g, w)
    ref = oracle.adam_step(p, m, v, g_full, sc)
    parts = []
    for lo in range(0, psi, bucket):
        hi = min(lo + bucket, psi)
        gb = oracle.reduce_full([x[lo:hi] for x in g], w)
        parts.append(oracle.adam_step(p[lo:hi], m[lo:hi], v[lo:hi], gb, sc))
    for i in range(4):
        assert np.array_equal(np.concatenate([q[i] for q in parts]).view(np.uint8),
                              ref[i].view(np.uint8))


def test_padding_is_inert():
    # padded elements carry zero gradient and zero state: without weight decay
    # they stay exactly zero after the step
    n, psi = 4, 1000
    _, pad, _ = oracle.shard_layout([psi], n)
    g, p, m, v, w = _setup(n, psi, 60)
    gp = [oracle.flatten_pad([x], pad) for x in g]
    pp, mp, vp = (oracle.flatten_pad([x], pad) for x in (p, m, v))
    _, p1, m1, v1, b = oracle.ddp_step(gp, w, pp, mp, vp, _sc(1))
    assert not p1[psi:].any() and not m1[psi:].any() and not v1[psi:].any() and not b[psi:].any()
    _, q1, _, _, _ = oracle.ddp_step(g, w, p, m, v, _sc(1))
    assert np.array_equal(p1[:psi], q1)


# ----------------------------------------------------------- scalar brute force
def _r(x: float) -> float:
    """Round a float64 to binary32 (struct packs with round-to-nearest-even).
    For +,-,*,/,sqrt of binary32 operands the float64 result rounded once to
    binary32 is the correctly rounded binary32 result (53 >= 2*24 + 2)."""
    try:
        return struct.unpack("f", struct.pack("f", x))[0]
    except OverflowError:
        return float("inf") if x > 0 else float("-inf")


def _scalar_reduce(xs, ws):
    a = _r(ws[0] * xs[0])
    for x, w in zip(xs[1:], ws[1:]):
        a = _r(a + _r(w * x))
    return a


def _scalar_adam(p, m, v, g, sc):
    d = {k: float(x) for k, x in sc.items()}
    m1 = _r(_r(d["beta1"] * m) + _r(d["one_minus_beta1"] * g))
    v1 = _r(_r(d["beta2"] * v) + _r(d["one_minus_beta2"] * _r(g * g)))
    mh = _r(m1 / d["bias_correction1"])
    vh = _r(v1 / d["bias_correction2"])
    u = _r(mh / _r(_r(vh ** 0.5) + d["eps"]))
    if d["weight_decay"] != 0.0:
        u = _r(u + _r(d["weight_decay"] * p))
    return _r(p - _r(d["lr"] * u)), m1, v1


@pytest.mark.parametrize("psi", [1, 255, 256, 1023, 1025, 4097])
@pytest.mark.parametrize("n", [1, 2, 3, 4, 8])
def test_scalar_brute_force(psi, n):
    psi_eff = min(psi, 300) if n == 8 else psi
    g, p, m, v, w = _setup(n, psi_eff, 70 + psi + n, counts=list(range(2, 2 + n)))
    sc = _sc(7, 0.1)
    gv, pv, mv, vv, _ = oracle.ddp_step(g, w, p, m, v, sc)
    xs = [oracle.bf16_to_f32(x).tolist() for x in g]
    ws = [float(x) for x in w]
    for i in range(psi_eff):
        gs = _scalar_reduce([x[i] for x in xs], ws)
        assert gs == float(gv[i])
        ps, ms, vs = _scalar_adam(float(p[i]), float(m[i]), float(v[i]), gs, sc)
        assert (ps, ms, vs) == (float(pv[i]), float(mv[i]), float(vv[i])), i


def test_elastic_reshard_is_concat_then_split():
    # the owners' state is a contiguous partition of one padded flat vector, so
    # moving from N to N' owners is concatenation, re-padding and re-splitting:
    # training N=4 for two steps, resharding to N'=2 and N'=8 and training a
    # third step with N' ranks equals the replicated run with those ranks
    psi = 3000
    n0 = 4
    _, pad0, _ = oracle.shard_layout([psi], n0)
    g0, p, m, v, w0 = _setup(n0, psi, 70, counts=[5, 3, 5, 2])
    flat = [oracle.flatten_pad([x], pad0) for x in (p, m, v)]
    gpad = [oracle.flatten_pad([x], pad0) for x in g0]
    owners = [[x[a:b] for a, b in (oracle.shard_bounds(pad0, n0, k) for k in range(n0))] for x in flat]
    rep = [x.copy() for x in flat]
    for t in (1, 2):
        outs, _ = oracle.sharded_step(gpad, w0, owners[0], owners[1], owners[2], _sc(t, 0.1))
        owners = [[o[1 + i] for o in outs] for i in range(3)]
        _, rep[0], rep[1], rep[2], _ = oracle.ddp_step(gpad, w0, rep[0], rep[1], rep[2], _sc(t, 0.1))
    for n1 in (2, 8):
        _, pad1, _ = oracle.shard_layout([psi], n1)
        state = [oracle.flatten_pad([np.concatenate(o)[:psi]], pad1) for o in owners]
        g1, _, _, _, w1 = _setup(n1, psi, 80 + n1, counts=list(range(2, 2 + n1)))
        g1p = [oracle.flatten_pad([x], pad1) for x in g1]
        sl = [oracle.shard_bounds(pad1, n1, k) for k in range(n1)]
        outs, view = oracle.sharded_step(g1p, w1, *[[x[a:b] for a, b in sl] for x in state], _sc(3, 0.1))
        ref = oracle.ddp_step(g1p, w1, *[oracle.flatten_pad([x[:psi]], pad1) for x in rep], _sc(3, 0.1))
        for i in range(3):
            got = np.concatenate([o[1 + i] for o in outs])
            assert np.array_equal(got[:psi].view(np.uint32), ref[1 + i][:psi].view(np.uint32)), (n1, i)
            assert not got[psi:].any()          # padding stays zero (zero gradient, zero state)
        assert np.array_equal(view[:psi], ref[4][:psi])
