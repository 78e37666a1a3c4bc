"""Plain CPU oracle for the ZeRO sharded update.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import this module.  The product path (the
HIP library and its Python binding) never imports, calls or links it, and this
module imports nothing from the product package.

What it computes, and where the pages define it
------------------------------------------------
Three web pages describe the method; they are cited by title and section:

* slide  "分担数据，与分担保存责任，是两个动作" (beats b0-b3, notes 原 N46-N48)
* essay  "把训练账本放进多张设备" (sections 从持久状态开始记账, 数据分工与保存分工,
  ZeRO-3 的一次完整计算)
* blog   "数据并行与 ZeRO：三级分片各省多少" (sections 每个参数 16 字节 with its
  byte equation, 三级分片 with its table, 分片放到 CPU：两个缓冲就够)

Arithmetic convention: every array operation below is ONE IEEE-754 binary32
operation rounded to nearest-even (numpy ufuncs on float32 arrays with
np.float32 scalars; there is no fused multiply-add in numpy, and np.sqrt and
np.divide are correctly rounded).  Dtypes are asserted so that numpy's scalar
promotion can never silently widen a step to float64.

Readings of points the pages leave open:
Adam is Kingma & Ba's bias-corrected form with eps outside the square root;
weight decay is decoupled and scaled by the learning rate; the reduction is
w_0*x_0 + w_1*x_1 + ... summed left to right in rank order with every product
and sum rounded separately; the partition is N contiguous equal slices of the
zero-padded flat vector; BF16 rounding is round-to-nearest-even.

Pins: every function here is checked by the CPU tests against values the
pages print, closed forms, exact rational arithmetic or an independent
library routine (see the tests named test_oracle_*).  Parity unpinned: the
exact bits of multi-step AdamW states beyond what the closed forms fix rest
on the readings above; the pins fix the formula, and a per-element scalar
evaluation fixes the vectorised code.
"""
from __future__ import annotations

import math
from fractions import Fraction
from typing import Iterable, Sequence

import numpy as np

F32 = np.float32
U16 = np.uint16
U32 = np.uint32

# Padding granularity per shard: every owner shard is a whole number of
# 256-element blocks (plain reading: the pages fix no padding rule).
SHARD_ALIGN = 256


def _f32(x) -> np.float32:
    return np.float32(x)


def _chk32(a: np.ndarray) -> np.ndarray:
    assert a.dtype == F32, a.dtype
    return a


# ---------------------------------------------------------------------------
# Flatten, pad, partition
# ---------------------------------------------------------------------------
def shard_layout(numels: Iterable[int], n_shards: int, align: int = SHARD_ALIGN):
    """Return (psi, psi_pad, shard_numel) for a unit made of tensors `numels`.

    The flat parameter vector is split into N owner shards theta_0..theta_{N-1}
    that are slices of the parameters, not layers (slide, note 原 N46).  Each
    owner holds 1/N of it (blog, section 三级分片).  psi_pad is psi rounded up
    to a multiple of N*align so that all shards are equal.
    """
    numels = [int(n) for n in numels]
    assert n_shards >= 1 and all(n >= 0 for n in numels)
    psi = sum(numels)
    q = n_shards * align
    psi_pad = ((psi + q - 1) // q) * q
    return psi, psi_pad, psi_pad // n_shards


def flatten_pad(tensors: Sequence[np.ndarray], psi_pad: int) -> np.ndarray:
    """Concatenate the unit's tensors in the stated order, zero-padded to psi_pad.

    The shards are slices of the flattened parameters, not layers (slide, note
    原 N46); the zero padding that makes the N slices equal is the reading
    taken where the pages are silent."""
    flat = np.concatenate([np.asarray(t).reshape(-1) for t in tensors]) if tensors else np.zeros(0)
    assert flat.size <= psi_pad
    out = np.zeros(psi_pad, dtype=flat.dtype)
    out[: flat.size] = flat
    return out


def shard_bounds(psi_pad: int, n_shards: int, k: int):
    """Owner k's contiguous slice [k*S, (k+1)*S) of the padded flat vector: each
    of the N devices keeps 1/N of the state (blog, section 三级分片; slide,
    note 原 N46, shards theta_0..theta_{N-1})."""
    assert psi_pad % n_shards == 0 and 0 <= k < n_shards
    s = psi_pad // n_shards
    return k * s, (k + 1) * s


# ---------------------------------------------------------------------------
# Loss-normalisation weights
# ---------------------------------------------------------------------------
def weights_mean(n_ranks: int) -> np.ndarray:
    """Equal weights 1/N: the batch-mean objective (slide, note 原 N48)."""
    return np.array([float(1) / float(n_ranks)] * n_ranks, dtype=np.float64).astype(F32)


def weights_from_counts(counts: Sequence[int]) -> np.ndarray:
    """w_r = n_r / sum(n), for ranks that saw different sample or token counts.

    The essay (section 数据分工与保存分工) says that blind equal averaging is
    wrong when counts differ; the slide (note 原 N48) says the reduction must be
    scaled to match the objective.  Each weight is the float64 quotient of the
    two integers, rounded once to float32.
    """
    counts = [int(c) for c in counts]
    assert all(c >= 0 for c in counts) and sum(counts) > 0
    total = float(sum(counts))
    return np.array([float(c) / total for c in counts], dtype=np.float64).astype(F32)


# ---------------------------------------------------------------------------
# BF16 encoding (definition: bfloat16 keeps the sign, the 8 exponent bits and
# the top 7 fraction bits of binary32)
# ---------------------------------------------------------------------------
def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening: a bf16 bit pattern is the high half of a binary32.  The
    working weights and gradients are 2-byte BF16 next to the 4-byte FP32
    master and moments (blog, section 每个参数 16 字节)."""
    bits = np.asarray(bits)
    assert bits.dtype == U16, bits.dtype
    return (bits.astype(U32) << U32(16)).view(F32)


def f32_to_bf16_rne(x: np.ndarray) -> np.ndarray:
    """Round binary32 values to the nearest bfloat16, ties to even mantissa.

    The BF16 working weight is derived from the FP32 master (blog, section
    每个参数 16 字节); the pages do not state a rounding mode, and
    round-to-nearest-even is the reading taken.

    Written from the definition: the two bf16 neighbours of |x| are the
    truncation `lo` and the next bf16 magnitude `hi` (the next bit pattern;
    past the largest finite value that is 2**128, which encodes as infinity).
    The distances are exact in float64 because both neighbours and x are
    binary32 numbers of nearly equal exponent.  NaN inputs give a quiet NaN.
    """
    x = np.asarray(x)
    assert x.dtype == F32, x.dtype
    with np.errstate(invalid="ignore", over="ignore"):
        return _f32_to_bf16_rne(x)


def _f32_to_bf16_rne(x: np.ndarray) -> np.ndarray:
    bits = x.view(U32)
    sign = (bits >> U32(16)) & U32(0x8000)
    mag = bits & U32(0x7FFFFFFF)
    is_nan = mag > U32(0x7F800000)
    is_inf = mag == U32(0x7F800000)
    lo = mag & U32(0xFFFF0000)
    hi = lo + U32(0x10000)
    xv = mag.view(F32).astype(np.float64)
    lo_v = lo.view(F32).astype(np.float64)
    hi_bits_f32 = np.where(hi >= U32(0x7F800000), U32(0), hi)  # avoid NaN/inf views
    hi_v = np.where(hi >= U32(0x7F800000), 2.0 ** 128, hi_bits_f32.view(F32).astype(np.float64))
    d_lo = xv - lo_v
    d_hi = hi_v - xv
    lo_odd = ((lo >> U32(16)) & U32(1)) == U32(1)
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & lo_odd)
    take_hi &= ~is_inf & ~is_nan
    res = np.where(take_hi, hi, lo) >> U32(16)
    res = np.where(is_nan, U32(0x7FC0), res)
    return (res | sign).astype(U16)


# ---------------------------------------------------------------------------
# Element-wise weighted reduction (all-reduce result) and reduce-scatter
# ---------------------------------------------------------------------------
def _contribution_f32(x: np.ndarray) -> np.ndarray:
    """A rank's contribution as float32: BF16 bit patterns are widened exactly;
    FP32 contributions (gradients stored in FP32, the blog's +2 bytes variant in
    section 每个参数 16 字节) are used as they are."""
    x = np.asarray(x)
    return bf16_to_f32(x) if x.dtype == U16 else _chk32(x)

def reduce_full(rank_grads: Sequence[np.ndarray], weights: np.ndarray) -> np.ndarray:
    """The combined gradient of every parameter: sum_r w_r * g_r, in FP32.

    Contributions of the same parameter are combined element-wise and never
    mixed with other parameters (slide, note 原 N48; essay, section ZeRO-3 的
    一次完整计算).  Order: a = w_0*x_0, then a = a + w_r*x_r for r = 1..N-1.
    """
    weights = np.asarray(weights)
    assert weights.dtype == F32 and len(rank_grads) == weights.size >= 1
    with np.errstate(all="ignore"):       # IEEE propagation of inf/NaN is intended
        a = _chk32(weights[0] * _contribution_f32(rank_grads[0]))
        for r in range(1, len(rank_grads)):
            term = _chk32(weights[r] * _contribution_f32(rank_grads[r]))
            a = _chk32(a + term)
    return a


def reduce_owner_shard(rank_grads: Sequence[np.ndarray], weights: np.ndarray,
                       n_shards: int, k: int) -> np.ndarray:
    """Reduce-scatter: owner k receives the reduction of its slice only.

    Each owner keeps the 1/N that matches its optimizer state (blog, section
    三级分片, ZeRO-2 paragraph).  Computed from owner k's slices alone.
    """
    weights = np.asarray(weights)
    assert weights.dtype == F32
    lo, hi = shard_bounds(rank_grads[0].size, n_shards, k)
    a = None
    for r, g in enumerate(rank_grads):
        term = _chk32(weights[r] * _contribution_f32(g[lo:hi]))
        a = term if a is None else _chk32(a + term)
    return a


def reduce_scatter(rank_grads, weights, n_shards: int):
    """Every owner's reduced shard: contributions combined element by element,
    each participant keeping its own fragment (essay, section ZeRO-3 的一次完整
    计算)."""
    return [reduce_owner_shard(rank_grads, weights, n_shards, k) for k in range(n_shards)]


def reduce_accumulate(acc: np.ndarray, rank_grads, weights) -> np.ndarray:
    """Accumulate mode: acc + (sum_r w_r x_r), the reduction formed first: a
    chunk reduced across the data ranks is added onto the accumulated shard
    (blog, section 分片放到 CPU：两个缓冲就够)."""
    _chk32(acc)
    return _chk32(acc + reduce_full(rank_grads, weights))


# ---------------------------------------------------------------------------
# Mixed-precision Adam owner update, BF16 working-weight pack
# ---------------------------------------------------------------------------
def adam_scalars(lr, beta1, beta2, eps, weight_decay, step: int) -> dict:
    """Per-step scalars, formed once on the host.  The pages name only Adam's
    two history statistics (essay, section 从持久状态开始记账); the bias
    corrections 1 - beta_i**t are those of Kingma & Ba's Algorithm 1.

    beta_i and the other hyper-parameters are rounded to float32; 1 - beta_i is
    a float32 subtraction (exact, since beta_i lies in [1/2, 1]); the bias
    corrections are 1 - beta_i**t evaluated in float64 from the float32 beta_i
    and rounded once to float32.
    """
    assert step >= 1
    b1, b2 = _f32(beta1), _f32(beta2)
    return {
        "lr": _f32(lr), "beta1": b1, "beta2": b2,
        "one_minus_beta1": _f32(F32(1) - b1),
        "one_minus_beta2": _f32(F32(1) - b2),
        "bias_correction1": _f32(1.0 - math.pow(float(b1), step)),
        "bias_correction2": _f32(1.0 - math.pow(float(b2), step)),
        "eps": _f32(eps), "weight_decay": _f32(weight_decay),
    }


def adam_step(master, exp_avg, exp_avg_sq, grad, sc: dict):
    """One Adam/AdamW update of an owner's FP32 master shard and its m/v.

    The owner updates its master weights and m/v with the combined gradient
    (slide, note 原 N48); FP32 master, first and second moments and a BF16
    working weight are the per-parameter state (essay, section 从持久状态开始
    记账; blog, section 每个参数 16 字节).  The update rule itself is Kingma &
    Ba's bias-corrected Adam with decoupled weight decay:

        m' = b1*m + (1-b1)*g
        v' = b2*v + (1-b2)*(g*g)
        u  = (m'/bc1) / (sqrt(v'/bc2) + eps)
        u  = u + wd*p            (only when wd != 0)
        p' = p - lr*u
        b  = bf16_rne(p')

    Returns (p', m', v', b).
    """
    p, m, v, g = (_chk32(np.asarray(a)) for a in (master, exp_avg, exp_avg_sq, grad))
    assert p.shape == m.shape == v.shape == g.shape
    for key, val in sc.items():
        assert type(val) is np.float32, key
    with np.errstate(all="ignore"):       # IEEE propagation of inf/NaN is intended
        return _adam_step(p, m, v, g, sc)


def _adam_step(p, m, v, g, sc):
    m1 = _chk32(_chk32(sc["beta1"] * m) + _chk32(sc["one_minus_beta1"] * g))
    gg = _chk32(g * g)
    v1 = _chk32(_chk32(sc["beta2"] * v) + _chk32(sc["one_minus_beta2"] * gg))
    m_hat = _chk32(m1 / sc["bias_correction1"])
    v_hat = _chk32(v1 / sc["bias_correction2"])
    denom = _chk32(np.sqrt(v_hat) + sc["eps"])
    u = _chk32(m_hat / denom)
    if sc["weight_decay"] != F32(0):
        u = _chk32(u + _chk32(sc["weight_decay"] * p))
    p1 = _chk32(p - _chk32(sc["lr"] * u))
    return p1, m1, v1, f32_to_bf16_rne(p1)


# ---------------------------------------------------------------------------
# All-gather into a temporary full view
# ---------------------------------------------------------------------------
def all_gather(shards: Sequence[np.ndarray], psi: int | None = None) -> np.ndarray:
    """Every participant's full view is the concatenation of the owner shards
    (essay, section ZeRO-3 的一次完整计算; slide, note 原 N47), cropped to the
    real parameter count."""
    full = np.concatenate(list(shards))
    return full if psi is None else full[:psi]


# ---------------------------------------------------------------------------
# Replicated data parallelism: the comparator the sharded path must equal
# ---------------------------------------------------------------------------
def ddp_step(rank_grads, weights, master, exp_avg, exp_avg_sq, sc: dict):
    """Unsharded, replicated DP: every replica all-reduces the full gradient and
    updates the full state (essay, section 数据分工与保存分工; blog, opening).
    Written without any sharding so the sharded path can be checked against it.
    """
    g = reduce_full(rank_grads, weights)
    p1, m1, v1, b = adam_step(master, exp_avg, exp_avg_sq, g, sc)
    return g, p1, m1, v1, b


def sharded_step(rank_grads, weights, masters, exp_avgs, exp_avg_sqs, sc: dict):
    """ZeRO-1/2 step as the pages describe it: reduce-scatter, each owner updates
    its shard, all-gather the BF16 shards (blog, section 三级分片, ZeRO-1
    paragraph; slide, note 原 N48).  Returns (grad shards, new states, view)."""
    n = len(masters)
    outs = []
    for k in range(n):
        g_k = reduce_owner_shard(rank_grads, weights, n, k)
        outs.append((g_k,) + adam_step(masters[k], exp_avgs[k], exp_avg_sqs[k], g_k, sc))
    view = all_gather([o[4] for o in outs])
    return outs, view


# ---------------------------------------------------------------------------
# Host-offloaded gradient shard accumulated over micro-batches
# ---------------------------------------------------------------------------
def offload_accumulate(per_micro_batch_grads: Sequence[Sequence[np.ndarray]], weights) -> np.ndarray:
    """The host gradient shard after M micro-batches (blog, section 分片放到
    CPU：两个缓冲就够): each chunk is reduced across the data ranks and added to
    the shard.  acc_1 = r_1, acc_m = acc_{m-1} + r_m."""
    acc = None
    for grads in per_micro_batch_grads:
        r = reduce_full(grads, weights)
        acc = r if acc is None else _chk32(acc + r)
    return acc


# ---------------------------------------------------------------------------
# Optional global gradient norm and clipping (not described by the pages; the
# plain reading: the Euclidean norm of the whole reduced gradient, and the
# gradient scaled by min(1, max_norm / (norm + 1e-6)) before the update)
# ---------------------------------------------------------------------------
def grad_norm_sq(shards: Sequence[np.ndarray]) -> float:
    """Sum of squares of every element of every shard, in float64 (the squares
    of binary32 values are exact in binary64).  Gradient clipping is not
    described by the pages; this is the plain reading of a global norm."""
    total = 0.0
    for x in shards:
        x64 = _chk32(np.asarray(x)).astype(np.float64)
        total += float(np.sum(x64 * x64))
    return total


def clip_coefficient(norm_sq: float, max_norm: float) -> np.float32:
    """float32(min(1, max_norm / (sqrt(norm_sq) + 1e-6))), evaluated in float64
    (not described by the pages: the plain reading of norm clipping)."""
    c = float(np.float32(max_norm)) / (math.sqrt(norm_sq) + 1e-6)
    return np.float32(min(1.0, c))


def scale_grad(g: np.ndarray, coef: np.float32) -> np.ndarray:
    """The clipped gradient: one binary32 multiply per element (not described by
    the pages: the plain reading of norm clipping)."""
    assert type(coef) is np.float32
    return _chk32(_chk32(np.asarray(g)) * coef)


# ---------------------------------------------------------------------------
# Ledger: persistent bytes per parameter (blog, 每个参数 16 字节 equation and
# the 三级分片 table; slide, note 原 N47; essay, 从持久状态开始记账)
# ---------------------------------------------------------------------------
WEIGHT_B, GRAD_B, MASTER_B, MOMENT_B = 2, 2, 4, 4


def ledger_bytes_per_param(stage: int, n: int, moments: int = 2, grad_bytes: int = GRAD_B) -> Fraction:
    """Persistent bytes per parameter per device (blog, section 每个参数 16 字节
    and the table of section 三级分片; slide, notes 原 N46 and 原 N47).

    stage 0 is replicated DP; stage 1 shards the optimizer state (master and
    moments); stage 2 also shards the gradient; stage 3 also shards the
    working weight.  `moments` = 2 for Adam, 1 for a first-moment-only
    optimizer; `grad_bytes` = 4 for FP32 gradient storage.
    """
    assert n >= 1 and stage in (0, 1, 2, 3)
    opt = Fraction(MASTER_B + moments * MOMENT_B)
    w, g = Fraction(WEIGHT_B), Fraction(grad_bytes)
    if stage >= 1:
        opt /= n
    if stage >= 2:
        g /= n
    if stage >= 3:
        w /= n
    return w + g + opt


def ledger_gb(stage: int, n: int, psi: int, **kw) -> Fraction:
    """Persistent state per device in GB (1 GB = 10**9 bytes), as the slide's
    note 原 N47 prints it for an 8B model on 4 cards."""
    return ledger_bytes_per_param(stage, n, **kw) * psi / 10 ** 9
