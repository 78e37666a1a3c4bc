"""Property-based versions of the invariants the pages state, over random rank
counts, sizes, count weights, steps and seeds (CPU only, hypothesis):

* sharded owners train the same model as replicated DP, and the gathered view
  is the one new version (slide, beat b3 and note 原 N48; essay, section ZeRO-3
  的一次完整计算);
* all-reduce equals reduce-scatter followed by all-gather (essay, section
  ZeRO-3 的一次完整计算; blog, section 三级分片);
* splitting the unit into buckets changes nothing (essay, section ZeRO-3 的一次
  完整计算, the bucketing paragraph);
* the offload accumulation over micro-batches equals the device-side
  accumulate-mode reduction (blog, section 分片放到 CPU：两个缓冲就够).
Every comparison is bit for bit."""
import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle
import synthetic as S

SETTINGS = settings(max_examples=40, deadline=None, suppress_health_check=[HealthCheck.too_slow])


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint32 if a.dtype == np.float32 else np.uint16)


@st.composite
def unit(draw):
    n = draw(st.integers(1, 8))
    blocks = draw(st.integers(1, 4))                 # shard = blocks * 256 elements
    psi = n * 256 * blocks
    counts = draw(st.lists(st.integers(1, 5000), min_size=n, max_size=n))
    seed = draw(st.integers(0, 2 ** 31 - 1))
    step = draw(st.sampled_from([1, 2, 3, 17, 1000]))
    wd = draw(st.sampled_from([0.0, 0.1]))
    return n, psi, counts, seed, step, wd


def _inputs(n, psi, counts, seed):
    g = S.rng(seed)
    grads = [S.bf16_normal(g, psi, 1e-3, float(g.uniform(0.5, 2.0))) for _ in range(n)]
    p, m, v = S.host_state(seed + 1, psi, 0.02, 1e-4, 1e-6)
    return grads, oracle.weights_from_counts(counts), p, m, v


@SETTINGS
@given(unit())
def test_sharded_equals_replicated_everywhere(u):
    n, psi, counts, seed, step, wd = u
    grads, w, p, m, v = _inputs(n, psi, counts, seed)
    sc = oracle.adam_scalars(1e-3, 0.9, 0.999, 1e-8, wd, step)
    gd, pd, md, vd, bd = oracle.ddp_step(grads, w, p, m, v, sc)
    sl = [oracle.shard_bounds(psi, n, k) for k in range(n)]
    outs, view = oracle.sharded_step(grads, w, [p[a:b] for a, b in sl], [m[a:b] for a, b in sl],
                                     [v[a:b] for a, b in sl], sc)
    for i, ref in enumerate((gd, pd, md, vd)):
        assert np.array_equal(_bits(np.concatenate([o[i] for o in outs])), _bits(ref)), i
    assert np.array_equal(view, bd)
    assert np.array_equal(view, oracle.f32_to_bf16_rne(np.concatenate([o[1] for o in outs])))


@SETTINGS
@given(unit())
def test_all_reduce_is_reduce_scatter_then_all_gather(u):
    n, psi, counts, seed, _, _ = u
    grads, w, _, _, _ = _inputs(n, psi, counts, seed)
    for n_shards in sorted({1, n, 2 * n}):
        if psi % n_shards:
            continue
        rs = oracle.reduce_scatter(grads, w, n_shards)
        assert np.array_equal(_bits(oracle.all_gather(rs)), _bits(oracle.reduce_full(grads, w)))


@SETTINGS
@given(unit(), st.integers(1, 3000))
def test_buckets_change_nothing(u, bucket):
    n, psi, counts, seed, step, wd = u
    grads, w, p, m, v = _inputs(n, psi, counts, seed)
    sc = oracle.adam_scalars(1e-3, 0.9, 0.999, 1e-8, wd, step)
    ref = oracle.adam_step(p, m, v, oracle.reduce_full(grads, w), sc)
    parts = [oracle.adam_step(p[lo:lo + bucket], m[lo:lo + bucket], v[lo:lo + bucket],
                              oracle.reduce_full([x[lo:lo + bucket] for x in grads], w), sc)
             for lo in range(0, psi, bucket)]
    for i in range(4):
        assert np.array_equal(_bits(np.concatenate([q[i] for q in parts])), _bits(ref[i])), i


@SETTINGS
@given(st.integers(1, 8), st.integers(1, 6), st.integers(1, 2000), st.integers(0, 2 ** 31 - 1))
def test_offload_accumulation_is_the_accumulate_mode_chain(n, n_micro, length, seed):
    g = S.rng(seed)
    mbs = [[S.bf16_normal(g, length, 1e-3) for _ in range(n)] for _ in range(n_micro)]
    w = np.full(n, 1.0 / (n * n_micro), np.float32)
    acc = oracle.reduce_full(mbs[0], w)
    for mb in mbs[1:]:
        acc = oracle.reduce_accumulate(acc, mb, w)
    assert np.array_equal(_bits(oracle.offload_accumulate(mbs, w)), _bits(acc))
