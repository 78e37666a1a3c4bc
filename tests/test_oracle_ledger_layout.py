"""Pins of the oracle's ledger, layout and weights against what the pages print
and what plain arithmetic fixes (CPU only)."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from synthetic import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ledger.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_bytes_per_param_printed_values():
    for e in _golden()["bytes_per_param"]:
        kw = {k: e[k] for k in ("moments", "grad_bytes") if k in e}
        assert oracle.ledger_bytes_per_param(e["stage"], e["n"], **kw) == e["value"], e["case"]


@pytest.mark.parametrize("n", [1, 2, 3, 4, 8, 16, 64])
def test_bytes_per_param_formulas(n):
    # the pages' table: 16, 4+12/N, 2+14/N, 16/N
    forms = {0: Fraction(16), 1: 4 + Fraction(12, n), 2: 2 + Fraction(14, n), 3: Fraction(16, n)}
    assert {e["stage"] for e in _golden()["bytes_per_param_formula"]} == set(forms)
    for stage, val in forms.items():
        assert oracle.ledger_bytes_per_param(stage, n) == val
    # the ZeRO-1 text form 2 + 2 + 12/N is the same number
    assert oracle.ledger_bytes_per_param(1, n) == 2 + 2 + Fraction(12, n)


def test_gb_per_device_printed_values():
    for e in _golden()["gb_per_device"]:
        assert oracle.ledger_gb(e["stage"], e["n"], e["psi"]) == e["value_gb"], e["case"]


def test_optimizer_share():
    full = oracle.ledger_bytes_per_param(0, 1)
    opt = full - oracle.WEIGHT_B - oracle.GRAD_B
    assert opt / full == Fraction(_golden()["fractions"][0]["value"])


def test_stages_monotone_and_n1_degenerate():
    for n in (2, 4, 8):
        vals = [oracle.ledger_bytes_per_param(s, n) for s in range(4)]
        assert vals == sorted(vals, reverse=True) and len(set(vals)) == 4
    # with one replica nothing is saved
    assert {oracle.ledger_bytes_per_param(s, 1) for s in range(4)} == {16}


@pytest.mark.parametrize("psi,n", [(0, 4), (1, 4), (1023, 4), (1024, 4), (1025, 4), (5, 3),
                                   (202_375_168, 4), (2_000_000_000, 4), (525_336_576, 4)])
def test_shard_layout_invariants(psi, n):
    p, pad, s = oracle.shard_layout([psi], n)
    assert p == psi and pad % (n * 256) == 0 and s * n == pad
    assert 0 <= pad - psi < n * 256


def test_layout_of_the_workloads():
    # parameter counts follow from the stated shapes
    d, f = 4096, 11008
    assert W.LAYER_7B.psi == 4 * d * d + 3 * d * f == 202_375_168
    psi, pad, s = oracle.shard_layout(W.unit_numels(W.layer_7b_tensors()), 4)
    assert pad == psi and s == 50_593_792          # already a multiple of 4*256
    units = W.llama8b_units()
    assert len(units) == 34
    layer = sum(W.unit_numels(units[1][1]))
    assert layer == 2 * 4096 * 4096 + 2 * 4096 * 1024 + 3 * 4096 * 14336 == 218_103_808
    assert W.CHAIN_8B.psi == 2 * 128256 * 4096 + 32 * layer == 8_029_995_008
    for _, t in units:
        psi, pad, s = oracle.shard_layout(W.unit_numels(t), 4)
        assert pad == psi
    # the 8B chain's persistent state at 16 B/param sharded 4 ways (ZeRO-3)
    assert oracle.ledger_bytes_per_param(3, 4) * W.CHAIN_8B.psi * 4 == 16 * W.CHAIN_8B.psi


def test_flatten_pad_and_bounds():
    a = np.arange(5, dtype=np.float32)
    b = np.arange(7, dtype=np.float32) + 10
    psi, pad, s = oracle.shard_layout([5, 7], 4, align=1)
    flat = oracle.flatten_pad([a, b], pad)
    assert pad == 12 and list(flat[:5]) == list(a) and list(flat[5:12]) == list(b)
    psi, pad, s = oracle.shard_layout([5, 7], 4)
    flat = oracle.flatten_pad([a, b], pad)
    assert flat.size == 1024 and not flat[12:].any()
    bounds = [oracle.shard_bounds(pad, 4, k) for k in range(4)]
    assert bounds[0][0] == 0 and bounds[-1][1] == pad
    assert all(bounds[k][1] == bounds[k + 1][0] for k in range(3))


def _round_f32_exact(q: Fraction) -> np.float32:
    """Correct rounding of a positive rational to binary32 (brute force)."""
    x = np.float32(float(q))
    best = x
    for cand in (np.nextafter(x, np.float32(0)), np.nextafter(x, np.float32(np.inf))):
        d_c, d_b = abs(Fraction(float(cand)) - q), abs(Fraction(float(best)) - q)
        if d_c < d_b or (d_c == d_b and (cand.view(np.uint32) & 1) == 0):
            best = cand
    return best


@pytest.mark.parametrize("counts", [[4096, 3072, 4096, 2048], [1, 2, 3], [7, 7, 7, 7, 7],
                                    [1, 0, 5], [123457, 99991, 31337, 65536]])
def test_count_weights_are_correctly_rounded_quotients(counts):
    w = oracle.weights_from_counts(counts)
    assert w.dtype == np.float32
    for c, wr in zip(counts, w):
        assert wr == _round_f32_exact(Fraction(c, sum(counts)))
    # they sum to one within the rounding of N terms
    assert abs(float(np.sum(w.astype(np.float64))) - 1.0) <= len(counts) * 2 ** -24


def test_mean_weights_power_of_two_exact():
    for n in (1, 2, 4, 8, 16):
        assert all(Fraction(float(x)) == Fraction(1, n) for x in oracle.weights_mean(n))
