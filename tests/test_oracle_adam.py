"""Pins of the oracle's Adam/AdamW owner update (CPU only).

The pages name Adam's two moment statistics and the FP32 master weight but not
the update formula; the oracle uses Kingma & Ba's bias-corrected Adam with
decoupled weight decay.  These tests pin it with closed forms that hold for
that method independently of how it is coded: the first step is sign descent,
a constant gradient keeps m_hat = g and v_hat = g^2 at every step, a zero
gradient decays the moments by beta1 and beta2, and decoupled decay shrinks p
by the factor (1 - lr*wd).
"""
import math

import numpy as np
import pytest

import oracle
import synthetic as S

U = 2.0 ** -24
HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0)


def _sc(step, **over):
    hp = dict(HP, **over)
    return oracle.adam_scalars(hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"], step)


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def _state(seed, n=4096, g_sigma=1e-3):
    g = S.rng(seed)
    p = S.normal_f32(g, n, 0.02)
    grad = S.normal_f32(g, n, g_sigma)
    z = np.zeros(n, np.float32)
    return p, z.copy(), z.copy(), grad


def test_scalars():
    sc = _sc(1)
    # 1 - beta is exact in float32 (Sterbenz), so it equals the float64 difference
    assert float(sc["one_minus_beta1"]) == 1.0 - float(np.float32(0.9))
    assert float(sc["one_minus_beta2"]) == 1.0 - float(np.float32(0.999))
    # at t = 1 the bias correction is 1 - beta
    assert sc["bias_correction1"] == sc["one_minus_beta1"]
    assert sc["bias_correction2"] == sc["one_minus_beta2"]
    sc = _sc(1000)
    # bias corrections use the float32 betas: 1 - b^t, rounded once
    b1, b2 = float(np.float32(0.9)), float(np.float32(0.999))
    assert abs(float(sc["bias_correction1"]) - (1 - b1 ** 1000)) <= U
    assert abs(float(sc["bias_correction2"]) - (1 - b2 ** 1000)) <= U * 0.64


def test_first_step_is_sign_descent():
    p, m, v, g = _state(1)
    p1, m1, v1, b = oracle.adam_step(p, m, v, g, _sc(1))
    lr, eps = float(np.float32(1e-3)), float(np.float32(1e-8))
    gd = _f64(g)
    expected = _f64(p) - lr * gd / (np.abs(gd) + eps)
    # u carries at most ~9 roundings; p' one more, plus the rounding of lr*u
    bound = 12 * U * lr * np.abs(gd) / (np.abs(gd) + eps) + U * np.abs(expected)
    assert np.all(np.abs(_f64(p1) - expected) <= bound)
    # the moments are (1-beta1) g and (1-beta2) g^2
    assert np.all(np.abs(_f64(m1) - (1 - float(np.float32(0.9))) * gd) <= U * np.abs(_f64(m1)))
    assert np.all(np.abs(_f64(v1) - (1 - float(np.float32(0.999))) * gd * gd) <= 2 * U * _f64(v1))


def test_eps_is_outside_the_square_root():
    # g = 1e-3: |g|/(|g|+eps) = 0.99999 but |g|/sqrt(g^2+eps) = 0.995
    p = np.zeros(8, np.float32)
    g = np.full(8, 1e-3, np.float32)
    p1, *_ = oracle.adam_step(p, p.copy(), p.copy(), g, _sc(1))
    assert np.allclose(_f64(p1), -1e-3 * 1e-3 / (1e-3 + 1e-8), rtol=1e-6)


@pytest.mark.parametrize("steps", [2, 5, 20])
def test_constant_gradient_keeps_unit_steps(steps):
    # with m = v = 0 and the same g each step, m_t = (1-b1^t) g and
    # v_t = (1-b2^t) g^2 exactly in real arithmetic, so every step moves p by
    # lr*g/(|g|+eps): p_T = p_0 - T*lr*g/(|g|+eps)
    p, m, v, g = _state(2, g_sigma=1e-2)
    p0 = _f64(p)
    for t in range(1, steps + 1):
        p, m, v, _ = oracle.adam_step(p, m, v, g, _sc(t))
    lr = float(np.float32(1e-3))
    gd = _f64(g)
    step = lr * gd / (np.abs(gd) + float(np.float32(1e-8)))
    expected = p0 - steps * step
    bound = steps * (4 * t * U * np.abs(step) + 2 * U * (np.abs(p0) + steps * np.abs(step)))
    assert np.all(np.abs(_f64(p) - expected) <= bound)


def test_zero_gradient_decays_moments_by_beta():
    # step 1 with g, step 2 with g = 0: m_2 = b1*(1-b1)*g, v_2 = b2*(1-b2)*g^2,
    # and the step-2 update is lr * (b1/(1+b1)) / sqrt(b2/(1+b2)) * sign(g)
    p, m, v, g = _state(3, g_sigma=1e-2)
    p1, m1, v1, _ = oracle.adam_step(p, m, v, g, _sc(1))
    p2, m2, v2, _ = oracle.adam_step(p1, m1, v1, np.zeros_like(g), _sc(2))
    b1, b2 = float(np.float32(0.9)), float(np.float32(0.999))
    gd = _f64(g)
    assert np.all(np.abs(_f64(m2) - b1 * (1 - b1) * gd) <= 3 * U * np.abs(_f64(m2)))
    assert np.all(np.abs(_f64(v2) - b2 * (1 - b2) * gd * gd) <= 5 * U * _f64(v2))
    ratio = (b1 / (1 + b1)) / math.sqrt(b2 / (1 + b2))
    assert abs(ratio - 0.67006) < 1e-4
    lr = float(np.float32(1e-3))
    step = _f64(p1) - _f64(p2)
    eps = float(np.float32(1e-8))
    expected = lr * (b1 / (1 + b1)) * gd / (np.abs(gd) * math.sqrt(b2 / (1 + b2)) + eps)
    assert np.allclose(step, expected, rtol=2e-5, atol=0)


def test_zero_gradient_without_decay_is_identity():
    p, _, _, _ = _state(4)
    z = np.zeros_like(p)
    for t in (1, 7, 1000):
        p1, m1, v1, b = oracle.adam_step(p, z, z, z, _sc(t))
        assert np.array_equal(p1.view(np.uint32), p.view(np.uint32))
        assert not m1.any() and not v1.any()
        assert np.array_equal(b, oracle.f32_to_bf16_rne(p))


def test_decoupled_weight_decay():
    # g = 0, wd > 0: p' = p * (1 - lr*wd); coupled L2 would instead give a
    # sign step of size lr
    p, _, _, _ = _state(5)
    z = np.zeros_like(p)
    p1, m1, v1, _ = oracle.adam_step(p, z, z, z, _sc(1, weight_decay=0.1))
    lr, wd = float(np.float32(1e-3)), float(np.float32(0.1))
    expected = _f64(p) * (1 - lr * wd)
    assert np.all(np.abs(_f64(p1) - expected) <= 3 * U * np.abs(_f64(p)))
    assert not m1.any() and not v1.any()
    # with a gradient the decay adds lr*wd*p on top of the sign step
    p, m, v, g = _state(6)
    p1, *_ = oracle.adam_step(p, m, v, g, _sc(1, weight_decay=0.1))
    gd = _f64(g)
    expected = _f64(p) - lr * (gd / (np.abs(gd) + 1e-8) + wd * _f64(p))
    assert np.all(np.abs(_f64(p1) - expected) <= 14 * U * lr + 2 * U * np.abs(_f64(p)))


def test_midrun_state_within_forward_error_of_float64():
    # sanity check at t = 1000 with nonzero moments: the float32 result stays
    # within a forward-error bound of the same update evaluated in float64
    g = S.rng(7)
    n = 1 << 14
    p = S.normal_f32(g, n, 0.02)
    m = S.normal_f32(g, n, 1e-4)
    v = np.abs(S.normal_f32(g, n, 1e-6))
    grad = S.normal_f32(g, n, 1e-3)
    sc = _sc(1000, weight_decay=0.1)
    p1, m1, v1, _ = oracle.adam_step(p, m, v, grad, sc)
    d = {k: float(x) for k, x in sc.items()}
    md = d["beta1"] * _f64(m) + d["one_minus_beta1"] * _f64(grad)
    vd = d["beta2"] * _f64(v) + d["one_minus_beta2"] * _f64(grad) ** 2
    mag_m = d["beta1"] * np.abs(_f64(m)) + d["one_minus_beta1"] * np.abs(_f64(grad))
    assert np.all(np.abs(_f64(m1) - md) <= 2 * U * mag_m)
    assert np.all(np.abs(_f64(v1) - vd) <= 3 * U * vd)
    den = np.sqrt(vd / d["bias_correction2"]) + d["eps"]
    ud = (md / d["bias_correction1"]) / den + d["weight_decay"] * _f64(p)
    pd = _f64(p) - d["lr"] * ud
    # relative error of the Adam ratio is amplified by |m|'s cancellation only
    # through m' (bounded above), so bound in terms of the magnitudes involved
    u_mag = (mag_m / d["bias_correction1"]) / den + d["weight_decay"] * np.abs(_f64(p))
    bound = 10 * U * d["lr"] * u_mag + 2 * U * np.abs(pd)
    assert np.all(np.abs(_f64(p1) - pd) <= bound)


def test_special_values_propagate():
    p = np.array([1.0, np.inf, np.nan, 0.0, -0.0, 1e-40], np.float32)
    g = np.array([np.nan, 1e-3, 1e-3, np.inf, 0.0, 1e-40], np.float32)
    z = np.zeros_like(p)
    p1, m1, v1, b = oracle.adam_step(p, z, z, g, _sc(1))
    assert np.isnan(p1[0]) and np.isnan(m1[0])
    assert np.isinf(p1[1]) or np.isnan(p1[1])
    assert np.isnan(p1[2])
    assert np.isnan(p1[3])              # inf/inf
    assert p1[4] == 0 and np.signbit(p1[4])   # -0 - lr*0 = -0
    # bf16 of a NaN is a NaN
    assert (int(b[0]) & 0x7FFF) > 0x7F80


# ----------------------------------------------------- optional gradient clipping
def test_grad_norm_sq_is_the_exact_sum_of_squares():
    from fractions import Fraction
    rng = np.random.default_rng(21)
    shards = [S.normal_f32(rng, 300, 1e-3) for _ in range(3)]
    exact = sum(Fraction(float(x)) ** 2 for s in shards for x in s)
    got = oracle.grad_norm_sq(shards)
    assert abs(Fraction(got) - exact) <= exact * Fraction(1, 10 ** 12)
    assert oracle.grad_norm_sq([np.array([3.0, 4.0], np.float32)]) == 25.0
    assert oracle.grad_norm_sq([np.full(1000, 0.5, np.float32)]) == 250.0
    assert oracle.grad_norm_sq([np.zeros(0, np.float32)]) == 0.0


def test_clip_coefficient_closed_forms():
    assert oracle.clip_coefficient(0.25, 1.0) == np.float32(1.0)          # norm 0.5 below the limit
    assert oracle.clip_coefficient(1.0, 1.0) == np.float32(1.0 / (1.0 + 1e-6))
    c = oracle.clip_coefficient(4.0, 1.0)                                 # norm 2: halve
    assert abs(float(c) - 0.5) < 1e-6
    # after clipping, the norm is max_norm (to within the eps and rounding)
    rng = np.random.default_rng(22)
    g = S.normal_f32(rng, 4096, 1.0)
    c = oracle.clip_coefficient(oracle.grad_norm_sq([g]), 2.0)
    assert abs(math.sqrt(oracle.grad_norm_sq([oracle.scale_grad(g, c)])) - 2.0) < 1e-5
    # scaling by 1 or a power of two is exact
    assert np.array_equal(oracle.scale_grad(g, np.float32(1.0)), g)
    assert np.array_equal(oracle.scale_grad(g, np.float32(0.25)), g / np.float32(4))


@pytest.mark.parametrize("steps", [3, 20])
def test_constant_gradient_adamw_is_an_affine_recurrence(steps):
    # AdamW with a constant g: the moments do not see the decay, so m_hat = g
    # and v_hat = g^2 at every step as above, and p follows
    #   p_t = a*p_{t-1} - c,  a = 1 - lr*wd,  c = lr*g/(|g|+eps)
    # whose solution is p_T = a^T p_0 - c (1 - a^T)/(1 - a).  Also
    # m_T = (1 - b1^T) g and v_T = (1 - b2^T) g^2.  Hyper-parameters of the
    # 7B-class layer's AdamW (lr 1e-3, wd 0.1), t = 1..T.
    p, m, v, g = _state(7, g_sigma=1e-2)
    p0 = _f64(p)
    for t in range(1, steps + 1):
        p, m, v, _ = oracle.adam_step(p, m, v, g, _sc(t, weight_decay=0.1))
    lr, wd, eps = float(np.float32(1e-3)), float(np.float32(0.1)), float(np.float32(1e-8))
    b1, b2 = float(np.float32(0.9)), float(np.float32(0.999))
    gd = _f64(g)
    a = 1.0 - lr * wd
    c = lr * gd / (np.abs(gd) + eps)
    expected = a ** steps * p0 - c * (1 - a ** steps) / (1 - a)
    # each step: the update direction carries about 4t roundings (the moments'
    # t-step recurrences) plus a dozen in the step itself, relative to lr; the
    # decay product and the final subtraction add 3 roundings of |p|; a <= 1
    # keeps earlier errors from growing
    pmax = np.abs(p0) + steps * np.abs(c)
    bound = steps * ((4 * steps + 14) * U * lr + 3 * U * pmax)
    assert np.all(np.abs(_f64(p) - expected) <= bound)
    assert np.all(np.abs(_f64(m) - (1 - b1 ** steps) * gd) <= 3 * steps * U * np.abs(gd))
    assert np.all(np.abs(_f64(v) - (1 - b2 ** steps) * gd * gd) <= 4 * steps * U * gd * gd)
    # the decay is visible: where the closed forms with and without decay
    # are far apart, the oracle is far from the one without
    no_decay = p0 - steps * c
    apart = np.abs(expected - no_decay) > 10 * bound
    assert apart.mean() > 0.5
    assert np.all(np.abs(_f64(p) - no_decay)[apart] > bound[apart])
