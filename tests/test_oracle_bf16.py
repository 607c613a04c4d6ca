"""Pins of the oracle's bf16 helpers against things other than itself:
torch's CPU float32->bfloat16 conversion (a library routine), exact rational
arithmetic (Python's Fraction) and the format facts the pages state."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _torch_bf16_bits(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_rne_matches_torch_on_structured_patterns(orc):
    # every high half (sign, exponent, 7-bit mantissa) x low halves that hit
    # below/at/above the half-way point, both parities
    hi = np.arange(0, 1 << 16, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x4000, 0xC000], dtype=np.uint32)
    bits = (hi[:, None] | lows[None, :]).ravel()
    x = bits.view(np.float32)
    finite = ~np.isnan(x)
    ours = orc.bf16_from_f32(x)
    ref = _torch_bf16_bits(x)
    assert np.array_equal(ours[finite], ref[finite])
    # NaN stays a quiet NaN with the sign kept
    nan_out = ours[~finite]
    assert np.all((nan_out & 0x7F80) == 0x7F80) and np.all((nan_out & 0x0040) != 0)
    assert np.array_equal(nan_out >> 15, (bits[~finite] >> 31).astype(np.uint16))


def test_rne_matches_torch_on_random_patterns(orc):
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 1 << 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    finite = ~np.isnan(x)
    assert np.array_equal(orc.bf16_from_f32(x)[finite], _torch_bf16_bits(x)[finite])


@pytest.mark.slow
def test_rne_matches_torch_exhaustive(orc):
    step = 1 << 26
    for start in range(0, 1 << 32, step):
        bits = np.arange(start, start + step, dtype=np.uint64).astype(np.uint32)
        x = bits.view(np.float32)
        finite = ~np.isnan(x)
        assert np.array_equal(orc.bf16_from_f32(x)[finite], _torch_bf16_bits(x)[finite])


def _bf16_value(bits):
    return float(np.array([bits << 16], dtype=np.uint32).view(np.float32)[0])


def _rne_fraction(x: Fraction) -> float:
    """Nearest bf16 by exhaustive neighbour search with exact rationals."""
    f = float(x)
    b = int(_torch_bf16_bits(np.array([f], np.float32))[0])
    cands = {b, (b + 1) & 0xFFFF, (b - 1) & 0xFFFF}
    best = None
    for c in cands:
        v = _bf16_value(c)
        if not np.isfinite(v):
            continue
        d = abs(Fraction(v) - x)
        key = (d, c & 1)  # ties: even mantissa (last bit 0) first
        if best is None or key < best[0]:
            best = (key, v)
    return best[1]


def test_direct_rne_of_double_matches_exact_rationals(orc):
    rng = np.random.default_rng(11)
    vals = list(rng.standard_normal(3000) * np.exp2(rng.integers(-20, 20, 3000)))
    # exact half-way points between bf16 neighbours, plus a hair either side
    for k in range(200):
        a = _bf16_value(int(rng.integers(0x3000, 0x4F00)))
        sp = orc.bf16_ulp(a)
        vals += [a + sp / 2, a + sp / 2 + sp * 2 ** -30, a + sp / 2 - sp * 2 ** -30]
    for v in vals:
        got = _bf16_value(orc.bf16_from_f64(v))
        assert got == _rne_fraction(Fraction(v)), v


def test_bf16_grid_facts(orc):
    # spacing 1/128 between 1 and 2 ([R] 'Why it matters', paper §2.1)
    assert orc.bf16_ulp(1.0) == 2 ** -7 and orc.bf16_ulp(1.99) == 2 ** -7
    assert orc.bf16_ulp(2.0) == 2 ** -6 and orc.bf16_ulp(0.75) == 2 ** -8
    # exp(0) = 1 is a bf16 value ([R] quiz explanation)
    assert _bf16_value(orc.bf16_from_f64(1.0)) == 1.0
    # 1 + 2^-8 is the half-way point above 1: ties to even -> 1
    assert orc.bf16_boundary_distance(1.0 + 2 ** -8) == 0.0
    assert _bf16_value(orc.bf16_from_f64(1.0 + 2 ** -8)) == 1.0
    assert _bf16_value(orc.bf16_from_f64(1.0 + 3 * 2 ** -8)) == 1.0 + 2 ** -6


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_worked_example_1(orc):
    g = _load("worked_example_1.json")
    terms = list(g["terms"])
    i = g["residual_index"]
    terms[i] = float(np.float32(terms[i]))  # the residual sits in an fp32 accumulator
    bits, exact = orc.bf16_round_of_sum(terms)
    got = _bf16_value(bits)
    assert got == g["expected_bf16"]
    assert abs(exact - g["exact_printed"]) < 1e-5
    assert round(got - exact, 4) == g["error_printed"]
    c = g["counter_case"]
    t2 = list(c["terms"]); t2[i] = float(np.float32(t2[i]))
    b2, ex2 = orc.bf16_round_of_sum(t2)
    assert _bf16_value(b2) == c["expected_bf16"]
    err2 = _bf16_value(b2) - ex2
    assert 0 < err2 < abs(g["error_printed"]) / 10  # small and of the opposite sign
    n = g["no_residual_case"]
    b3, _ = orc.bf16_round_of_sum(n["terms"])
    assert _bf16_value(b3) == n["expected_bf16"]


def test_worked_example_1_needs_a_wide_accumulator(orc):
    """Rounding to bf16 after every addition loses the residual and gives
    -4.6875, not the page's -4.71875: the page's value pins accumulate-then-round."""
    g = _load("worked_example_1.json")
    t = [float(np.float32(x)) for x in g["terms"]]
    acc = 0.0
    for x in t:
        acc = _bf16_value(orc.bf16_from_f64(acc + x))
    assert acc == -4.6875 != g["expected_bf16"]


def test_worked_example_2(orc):
    g = _load("worked_example_2.json")
    bits, exact = orc.bf16_round_of_sum(g["terms"])
    got = _bf16_value(bits)
    assert got == g["expected_bf16"]
    assert exact == g["exact_printed"]
    assert abs(got - exact) == g["abs_error"]


def test_pair_enumeration_bias(orc):
    """[R] 'Core idea' (paper §3.3.2, App. B): adding two same-exponent bf16
    values (the P̄ = 1 terms) plus a small same-sign residual rounds away from
    zero whenever the pushed-out bit is 1.  Over every pair in [-4, -2) the
    mean error is -spacing/4 + |r| (half the sums are half-way points)."""
    # every bf16 value in (-4, -2]: bit patterns 0xC000 (-2) .. 0xC07F
    vals = sorted(set(v for v in (_bf16_value(b) for b in range(0xC000, 0xC081)) if -4 < v <= -2))
    assert len(vals) == 128
    r = float(np.float32(-0.00087))
    errs = []
    for a in vals:
        for b in vals:
            bits, exact = orc.bf16_round_of_sum([a, r, b])
            errs.append(_bf16_value(bits) - exact)
    errs = np.array(errs)
    spacing = 2 ** -5  # sums lie in (-8, -4]
    closed = -spacing / 4 + abs(r)
    assert errs.mean() < 0
    # exact closed form up to the (-4,-2] endpoint pairs whose sum is -4 (on the grid of [2,4))
    assert abs(errs.mean() - closed) < 2e-4
    assert np.mean(errs < 0) == pytest.approx(0.5, abs=0.01)


def test_random_pbar_has_no_bias(orc):
    """[R] 'Core idea' (paper §3.3.2 Remark 1): with P̄ < 1 the products fill
    the low bits and the rounding error averages out."""
    rng = np.random.default_rng(5)
    errs = []
    r = float(np.float32(-0.00087))
    for _ in range(20000):
        pa, pb = (_bf16_value(orc.bf16_from_f64(x)) for x in rng.uniform(0.5, 1.0, 2))
        va, vb = (_bf16_value(orc.bf16_from_f64(x)) for x in rng.uniform(-4, -2, 2))
        bits, exact = orc.bf16_round_of_sum([pa * va, r, pb * vb])
        errs.append((_bf16_value(bits) - exact) / orc.bf16_ulp(exact))
    errs = np.array(errs)
    assert abs(errs.mean()) < 0.01  # in ulps of the result; the P̄ = 1 case gives -0.22
