"""Pins of the oracle's BF16 encoding and its reduction (CPU only).

BF16 rounding is pinned against torch's own float32->bfloat16 conversion (a
library routine); the reduction against exact rational sums within the
recursive-summation error bound, and against special cases whose result is
fixed by the arithmetic alone.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synthetic as S

U = 2.0 ** -24


def _torch_bf16_bits(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _is_bf16_nan(b):
    return (b & 0x7FFF) > 0x7F80


def _check_rne_against_torch(bits32: np.ndarray):
    x = bits32.view(np.float32)
    ours = oracle.f32_to_bf16_rne(x)
    ref = _torch_bf16_bits(x)
    nan = np.isnan(x)
    assert np.array_equal(_is_bf16_nan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_bf16_rne_structured_sweep():
    # every sign/exponent/7-bit-mantissa prefix, with low halves that probe the
    # tie (0x8000), just below/above it, zero, the extremes and random values
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x4000, 0xC000],
                    dtype=np.uint32)
    lows = np.concatenate([lows, np.random.default_rng(5).integers(0, 1 << 16, 8, dtype=np.uint32)])
    _check_rne_against_torch((hi[:, None] | lows[None, :]).reshape(-1))


def _check_rne_range(start: int, count: int) -> int:
    """One worker's share of the exhaustive sweep; returns patterns checked."""
    torch.set_num_threads(1)
    _check_rne_against_torch(np.arange(start, start + count, dtype=np.uint64).astype(np.uint32))
    return count


def test_bf16_rne_all_2_32_patterns():
    # every binary32 bit pattern, in 2^24-pattern pieces over a process pool
    # (about 3.5 s of one core per 2^26 patterns)
    import concurrent.futures as cf
    import multiprocessing as mp
    import os
    step = 1 << 24
    starts = list(range(0, 1 << 32, step))
    workers = max(1, min(8, len(os.sched_getaffinity(0))))
    with cf.ProcessPoolExecutor(workers, mp_context=mp.get_context("spawn")) as ex:
        done = sum(ex.map(_check_rne_range, starts, [step] * len(starts)))
    assert done == 1 << 32


def test_bf16_rne_named_cases():
    f = lambda v: int(oracle.f32_to_bf16_rne(np.array([v], np.float32))[0])
    assert f(1.0) == 0x3F80 and f(-2.0) == 0xC000 and f(0.0) == 0 and f(-0.0) == 0x8000
    # 1 + 2^-8 is exactly halfway between 1 and 1 + 2^-7: ties to even (1.0)
    assert f(1.0 + 2 ** -8) == 0x3F80
    # 1 + 3*2^-8 is halfway between 1+2^-7 (odd) and 1+2^-6: rounds up to even
    assert f(1.0 + 3 * 2 ** -8) == 0x3F82
    assert f(float(np.finfo(np.float32).max)) == 0x7F80       # overflows to +inf
    assert f(np.inf) == 0x7F80 and f(-np.inf) == 0xFF80
    tiny = np.array([1], np.uint32).view(np.float32)[0]        # smallest subnormal
    assert f(tiny) == 0


def test_bf16_widening_exhaustive():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = oracle.bf16_to_f32(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_single_rank_unit_weight_is_exact_widening():
    g = S.host_rank_grads(11, 1, 4096)
    out = oracle.reduce_full(g, np.array([1.0], np.float32))
    ref = torch.from_numpy(g[0].view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(out.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("n", [2, 4, 8, 16])
def test_power_of_two_weights_commute_with_rounding(n):
    g = S.host_rank_grads(12, n, 8192)
    a = oracle.reduce_full(g, oracle.weights_mean(n))
    b = oracle.reduce_full(g, np.ones(n, np.float32)) * np.float32(1.0 / n)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 8])
def test_weighted_reduce_within_summation_bound_of_exact(n):
    rng = np.random.default_rng(100 + n)
    psi = 64 * n
    g = [S.bf16_normal(rng, psi, 1e-3, float(rng.uniform(0.5, 2.0))) for _ in range(n)]
    counts = list(rng.integers(1, 5000, n))
    w = oracle.weights_from_counts(counts)
    a = oracle.reduce_full(g, w)
    xs = [oracle.bf16_to_f32(x) for x in g]
    gamma = n * U / (1 - n * U)
    for i in range(psi):
        terms = [Fraction(float(w[r])) * Fraction(float(xs[r][i])) for r in range(n)]
        exact = sum(terms)
        bound = gamma * float(sum(abs(t) for t in terms))
        assert abs(float(Fraction(float(a[i])) - exact)) <= bound, (i, n)
    # reduce-scatter: owner k's shard matches the same exact sums at its global indices
    for k in range(n):
        lo, hi = oracle.shard_bounds(psi, n, k)
        sk = oracle.reduce_owner_shard(g, w, n, k)
        assert sk.size == hi - lo
        for j in (0, sk.size // 2, sk.size - 1):
            i = lo + j
            exact = sum(Fraction(float(w[r])) * Fraction(float(xs[r][i])) for r in range(n))
            assert abs(float(Fraction(float(sk[j])) - exact)) <= gamma * float(
                sum(abs(Fraction(float(w[r])) * Fraction(float(xs[r][i]))) for r in range(n)))


@pytest.mark.parametrize("n", [1, 3, 4])
def test_fp32_contributions_within_summation_bound_of_exact(n):
    rng = np.random.default_rng(300 + n)
    psi = 128 * n
    g = [S.normal_f32(rng, psi, 1e-3, float(rng.uniform(0.5, 2.0))) for _ in range(n)]
    w = oracle.weights_from_counts(list(rng.integers(1, 5000, n)))
    a = oracle.reduce_full(g, w)
    gamma = n * U / (1 - n * U)
    for i in range(0, psi, 7):
        terms = [Fraction(float(w[r])) * Fraction(float(g[r][i])) for r in range(n)]
        assert abs(float(Fraction(float(a[i])) - sum(terms))) <= gamma * float(sum(abs(t) for t in terms))
    # BF16-valued FP32 contributions reduce exactly like the BF16 bit patterns
    gb = [S.to_bf16_bits(x) for x in g]
    assert np.array_equal(oracle.reduce_full([oracle.bf16_to_f32(x) for x in gb], w).view(np.uint32),
                          oracle.reduce_full(gb, w).view(np.uint32))


def test_reduce_exact_when_representable():
    # small integers scaled by 2^-10 with power-of-two weights: every partial
    # sum is representable, so the reduction is the exact value
    rng = np.random.default_rng(3)
    n, psi = 4, 2048
    ints = [rng.integers(-100, 100, psi) for _ in range(n)]
    g = [S.to_bf16_bits((x * 2.0 ** -10).astype(np.float32)) for x in ints]
    a = oracle.reduce_full(g, oracle.weights_mean(n))
    exact = sum(ints).astype(np.float64) * 2.0 ** -10 / n
    assert np.array_equal(a.astype(np.float64), exact)


def test_rank_order_is_left_to_right():
    # (1 + 2^-24) + 2^-24 ... : summation order changes the result; rank order fixes it
    x = [np.array([v], np.float32) for v in (1.0, 2.0 ** -8, 2.0 ** -8, -1.0)]
    g = [S.to_bf16_bits(v) for v in x]
    w = np.array([1.0, 2.0 ** -16, 2.0 ** -16, 1.0], np.float32)
    a = oracle.reduce_full(g, w)
    # left to right: 1 + 2^-24 -> 1 (tie to even), + 2^-24 -> 1, - 1 -> 0
    assert a[0] == 0.0
    # a different order (the two small terms first) would give 2^-23
    assert np.float32(np.float32(np.float32(2.0 ** -24) + np.float32(2.0 ** -24)) + np.float32(1.0)) - np.float32(1.0) == np.float32(2.0 ** -23)


def test_allreduce_equals_reduce_scatter_then_all_gather():
    # the essay's identity (section ZeRO-3 的一次完整计算): all-reduce is
    # reduce-scatter followed by all-gather, in result
    for n in (1, 2, 3, 4, 8):
        g = S.host_rank_grads(20 + n, n, n * 256 * 3, scales=np.linspace(0.5, 2, n))
        w = oracle.weights_from_counts(list(range(1, n + 1)))
        ar = oracle.reduce_full(g, w)
        ag = oracle.all_gather(oracle.reduce_scatter(g, w, n))
        assert np.array_equal(ar.view(np.uint32), ag.view(np.uint32))


def test_accumulate_mode():
    g1 = S.host_rank_grads(30, 4, 1024)
    g2 = S.host_rank_grads(31, 4, 1024)
    w = oracle.weights_mean(4)
    acc = oracle.reduce_full(g1, w)
    acc2 = oracle.reduce_accumulate(acc, g2, w)
    assert np.array_equal(acc2, acc + oracle.reduce_full(g2, w))
    assert np.array_equal(oracle.offload_accumulate([g1, g2], w), acc2)


def test_offload_accumulation_exact_mean():
    # M micro-batches x N ranks of exactly representable contributions with
    # weights 1/(N*M): the accumulated shard is the exact mean of all of them
    rng = np.random.default_rng(9)
    n, m_count, psi = 4, 4, 4096
    ints = [[rng.integers(-64, 64, psi) for _ in range(n)] for _ in range(m_count)]
    grads = [[S.to_bf16_bits((x * 2.0 ** -6).astype(np.float32)) for x in mb] for mb in ints]
    w = np.full(n, 1.0 / (n * m_count), np.float32)
    acc = oracle.offload_accumulate(grads, w)
    exact = sum(sum(mb) for mb in ints).astype(np.float64) * 2.0 ** -6 / (n * m_count)
    assert np.array_equal(acc.astype(np.float64), exact)
