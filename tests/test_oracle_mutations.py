"""Plants plausible mistakes in a copy of the oracle, on the CPU, and checks that
the oracle's pins (not the scalar brute force, which restates the formulas)
catch every one of them.  Mistakes are planted in the oracle's arithmetic
(zero_oracle.py) and in the distance measures every parity test uses
(compare.py).  The pins run in a scratch tree holding the copy, the
tests and the input generators only; a control run on the unmodified copy must
pass there, and a planted mistake counts as caught only when a pin fails (an
error in collection or set-up does not count)."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTATIONS = {
    "no_bias_correction_m": ('m_hat = _chk32(m1 / sc["bias_correction1"])', 'm_hat = _chk32(m1 / F32(1))'),
    "eps_inside_sqrt": ('denom = _chk32(np.sqrt(v_hat) + sc["eps"])', 'denom = _chk32(np.sqrt(v_hat + sc["eps"]))'),
    "beta2_in_first_moment": ('m1 = _chk32(_chk32(sc["beta1"] * m) + _chk32(sc["one_minus_beta1"] * g))',
                              'm1 = _chk32(_chk32(sc["beta2"] * m) + _chk32(sc["one_minus_beta2"] * g))'),
    "wrong_decay_factor": ('m1 = _chk32(_chk32(sc["beta1"] * m)', 'm1 = _chk32(_chk32(sc["beta2"] * m)'),
    "weight_decay_dropped": ('u = _chk32(u + _chk32(sc["weight_decay"] * p))', 'u = u'),
    "update_sign": ('p1 = _chk32(p - _chk32(sc["lr"] * u))', 'p1 = _chk32(p + _chk32(sc["lr"] * u))'),
    "bias_correction1_exponent": ("math.pow(float(b1), step)", "math.pow(float(b1), step + 1)"),
    "bias_correction2_exponent": ("math.pow(float(b2), step)", "math.pow(float(b2), step - 1 if step > 1 else 1)"),
    "second_moment_not_squared": ("gg = _chk32(g * g)", "gg = _chk32(np.abs(g))"),
    "last_rank_dropped": ("for r in range(1, len(rank_grads)):", "for r in range(1, len(rank_grads) - 1):"),
    "owner_slice_shifted": ("    lo, hi = shard_bounds(rank_grads[0].size, n_shards, k)\n",
                            "    lo, hi = shard_bounds(rank_grads[0].size, n_shards, k)\n"
                            "    lo, hi = (lo + 1, hi + 1) if hi < rank_grads[0].size else (lo, hi)\n"),
    "weight_paired_with_wrong_rank": ("term = _chk32(weights[r] * _contribution_f32(rank_grads[r]))",
                                      "term = _chk32(weights[(r + 1) % len(rank_grads)] * _contribution_f32(rank_grads[r]))"),
    "bf16_ties_away": ("take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & lo_odd)", "take_hi = (d_hi <= d_lo)"),
    "bf16_truncates": ("take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & lo_odd)", "take_hi = d_hi < 0"),
    "bf16_widen_shift": ("<< U32(16)).view(F32)", "<< U32(15)).view(F32)"),
    "count_weights_off": ("total = float(sum(counts))", "total = float(sum(counts) + 1)"),
    "ledger_stage2_grad_unsharded": ("    if stage >= 2:\n        g /= n", "    if stage >= 3:\n        g /= n"),
    "padding_rule": ("psi_pad = ((psi + q - 1) // q) * q", "psi_pad = ((psi + q) // q) * q"),
    "gather_order": ("full = np.concatenate(list(shards))", "full = np.concatenate(list(shards)[::-1])"),
    "offload_not_accumulated": ("acc = r if acc is None else _chk32(acc + r)", "acc = r"),
    "norm_not_squared": ("total += float(np.sum(x64 * x64))", "total += float(np.sum(np.abs(x64)))"),
    "clip_uses_norm_sq": ("c = float(np.float32(max_norm)) / (math.sqrt(norm_sq) + 1e-6)",
                          "c = float(np.float32(max_norm)) / (norm_sq + 1e-6)"),
    "reversed_rank_order": ("        a = _chk32(weights[0] * _contribution_f32(rank_grads[0]))\n"
                            "        for r in range(1, len(rank_grads)):",
                            "        a = _chk32(weights[-1] * _contribution_f32(rank_grads[-1]))\n"
                            "        for r in range(len(rank_grads) - 2, -1, -1):"),
    "owner_shard_reversed_rank_order": ("    for r, g in enumerate(rank_grads):\n        term = _chk32(weights[r] * _contribution_f32(g[lo:hi]))",
                                        "    for r, g in reversed(list(enumerate(rank_grads))):\n"
                                        "        term = _chk32(weights[r] * _contribution_f32(g[lo:hi]))"),
    "decay_not_scaled_by_lr": ('u = _chk32(u + _chk32(sc["weight_decay"] * p))',
                               'u = _chk32(u + _chk32(_chk32(sc["weight_decay"] / sc["lr"]) * p))'),
    "coupled_l2_decay": ("def _adam_step(p, m, v, g, sc):\n    m1 =",
                         "def _adam_step(p, m, v, g, sc):\n"
                         "    g = _chk32(g + _chk32(sc[\"weight_decay\"] * p)) if sc[\"weight_decay\"] != F32(0) else g\n"
                         "    m1 ="),
    "bf16_packed_from_old_master": ("return p1, m1, v1, f32_to_bf16_rne(p1)", "return p1, m1, v1, f32_to_bf16_rne(p)"),
    "mean_weight_off": ("[float(1) / float(n_ranks)]", "[float(1) / float(n_ranks + 1)]"),
    "decay_also_on_first_moment": ('m1 = _chk32(_chk32(sc["beta1"] * m) + _chk32(sc["one_minus_beta1"] * g))',
                                   'm1 = _chk32(_chk32(_chk32(sc["beta1"] * m) + _chk32(sc["one_minus_beta1"] * g))'
                                   ' - _chk32(_chk32(sc["lr"] * sc["weight_decay"]) * m))'),
    "accumulate_mode_drops_acc": ("return _chk32(acc + reduce_full(rank_grads, weights))",
                                  "return _chk32(reduce_full(rank_grads, weights))"),
}

# Mistakes in the ulp distance and bit-equality measures: each would let a GPU
# result that is not the oracle's pass (or a correct one fail).
COMPARE_MUTATIONS = {
    "sign_map_dropped": ("return np.where(b & sign_bit, -mag, mag)", "return mag"),
    "sign_map_keeps_sign_bit": ("return np.where(b & sign_bit, -mag, mag)", "return np.where(b & sign_bit, -b, b)"),
    "two_nans_infinitely_apart": ("d = np.where(a_nan & b_nan, 0, d)", "d = np.where(a_nan & b_nan, INF_ULP, d)"),
    "nan_vs_number_not_infinite": ("d = np.where(a_nan ^ b_nan, INF_ULP, d)", "d = np.where(a_nan ^ b_nan, d, d)"),
    "f32_magnitude_mask_fraction_only": ("0x80000000, 0x7FFFFFFF)", "0x80000000, 0x007FFFFF)"),
    "bf16_infinity_taken_as_nan": ("a_nan = (a & 0x7FFF) > 0x7F80", "a_nan = (a & 0x7FFF) >= 0x7F80"),
    "bf16_nan_threshold_high": ("b_nan = (b & 0x7FFF) > 0x7F80", "b_nan = (b & 0x7FFF) > 0x7FC0"),
    "bf16_magnitude_mask_wrong": ("0x8000, 0x7FFF)", "0x8000, 0x7F80)"),
    "bits_equal_by_value": ("same = a.view(np.uint32) == b.view(np.uint32)", "same = a == b"),
    "bits_equal_nan_rule_dropped": ("same |= np.isnan(a) & np.isnan(b)", "pass"),
    "max_ulp_reports_min": ("return int(ulp_f32(a, b).max(initial=0))", "return int(ulp_f32(a, b).min(initial=0))"),
}

# the pin files; the scalar brute force restates the formulas, so it is left
# out, and the exhaustive 2^32 rounding sweep is left out for time (the
# structured sweep over every sign/exponent/mantissa prefix runs instead)
PIN_FILES = ["tests/test_oracle_adam.py", "tests/test_oracle_invariants.py",
             "tests/test_oracle_ledger_layout.py", "tests/test_oracle_reduce_bf16.py",
             "tests/test_oracle_compare.py"]


def _src(name):
    with open(os.path.join(ROOT, "oracle", name)) as f:
        return f.read()


@pytest.fixture(scope="module")
def oracle_src():
    return _src("zero_oracle.py")


@pytest.fixture(scope="module")
def compare_src():
    return _src("compare.py")


def _run_pins(tmp_path, src, name="zero_oracle.py"):
    shutil.copytree(os.path.join(ROOT, "oracle"), tmp_path / "oracle",
                    ignore=shutil.ignore_patterns("__pycache__"))
    (tmp_path / "oracle" / name).write_text(src)
    for d in ("tests", "synthetic"):
        os.symlink(os.path.join(ROOT, d), tmp_path / d)
    return subprocess.run(
        [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", *PIN_FILES,
         "-m", "not gpu", "-k", "not brute and not all_2_32"],
        cwd=tmp_path, capture_output=True, text=True, timeout=300)


def test_pins_pass_on_the_unmodified_oracle(oracle_src, tmp_path):
    r = _run_pins(tmp_path, oracle_src)
    assert r.returncode == 0, f"the pins fail on the unmodified copy:\n{r.stdout[-2000:]}"


def _assert_caught(name, r):
    last = r.stdout.strip().splitlines()[-1] if r.stdout.strip() else ""
    assert r.returncode == 1 and " failed" in last and " error" not in last, \
        f"planted mistake {name} was not caught by a failing pin:\n{r.stdout[-2000:]}"


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, oracle_src, tmp_path):
    old, new = MUTATIONS[name]
    assert old in oracle_src, f"mutation anchor for {name} no longer in the oracle"
    _assert_caught(name, _run_pins(tmp_path, oracle_src.replace(old, new, 1)))


@pytest.mark.parametrize("name", sorted(COMPARE_MUTATIONS))
def test_pins_catch_planted_mistake_in_the_distance_measures(name, compare_src, tmp_path):
    old, new = COMPARE_MUTATIONS[name]
    assert old in compare_src, f"mutation anchor for {name} no longer in compare.py"
    _assert_caught(name, _run_pins(tmp_path, compare_src.replace(old, new, 1), "compare.py"))
