"""Pins of the oracle's scalar references: exp_ref / sigmoid_ref / silu_ref and
the bf16 rounding helpers, against high-precision constants, fp64 libm and
torch's bf16 conversion."""
import math
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tests import refmath

getcontext().prec = 80


_rn32 = refmath.rn32


LN2 = Fraction(Decimal("0.69314718055994530941723212145817656807550013436025525412068000949339362"))
LOG2E = Fraction(Decimal("1.44269504088896340735992468100189213742664595415298593413544940693110921"))


def test_exp_constants_are_nearest_binary32():
    hi = _rn32(LN2)
    assert oracle.const(0) == _rn32(LOG2E)
    assert oracle.const(1) == hi
    assert oracle.const(2) == _rn32(LN2 - Fraction(hi))
    for m in range(8):
        assert oracle.const(3 + m) == _rn32(Fraction(1, math.factorial(m))), m


def _ulp32(x):
    x = np.abs(np.asarray(x, dtype=np.float32))
    return (np.nextafter(x, np.float32(np.inf)) - x).astype(np.float64)


def test_exp_ref_within_two_ulp_of_libm():
    g = np.random.default_rng(0)
    t = np.concatenate([
        np.linspace(-80, 80, 400001, dtype=np.float32),
        g.uniform(-80, 80, 400000).astype(np.float32),
        np.array([0.0, -0.0, 1e-30, -1e-30, 0.5, -0.5, 88.0 / 1.1, -80.0], np.float32),
    ])
    got = oracle.exp_ref_n(t).astype(np.float64)
    ref = np.exp(t.astype(np.float64))
    err_ulp = np.abs(got - ref) / _ulp32(ref.astype(np.float32))
    assert err_ulp.max() <= 2.0, float(err_ulp.max())
    assert oracle.exp_ref(0.0) == 1.0


def test_sigmoid_ref_accuracy_symmetry_monotone():
    z = np.linspace(-90, 90, 600001, dtype=np.float32)
    s = oracle.sigmoid_ref_n(z).astype(np.float64)
    zc = np.clip(z.astype(np.float64), -80, 80)
    ref = 1.0 / (1.0 + np.exp(-zc))
    err_ulp = np.abs(s - ref) / _ulp32(ref.astype(np.float32))
    assert err_ulp.max() <= 3.0, float(err_ulp.max())
    assert np.all(np.diff(s) >= 0)  # monotone: selection by score agrees with selection by logit
    s_neg = oracle.sigmoid_ref_n(-z).astype(np.float64)
    assert np.max(np.abs(s + s_neg - 1.0)) <= 2 ** -22
    assert oracle.sigmoid_ref(0.0) == 0.5
    assert np.all(s > 0) and np.all(s <= 1)


def test_silu_ref_accuracy():
    z = np.linspace(-60, 60, 300001, dtype=np.float32)
    got = oracle.silu_ref_n(z).astype(np.float64)
    ref = refmath.silu64(z)
    tol = 4 * _ulp32(ref.astype(np.float32)) + 1e-37
    assert np.all(np.abs(got - ref) <= tol)


def test_f32_to_bf16_matches_torch():
    g = np.random.default_rng(1)
    v = np.concatenate([
        g.standard_normal(200000).astype(np.float32) * np.float32(10.0) ** g.integers(-20, 20, 200000).astype(np.float32),
        np.array([1.0, -1.0, 0.0, -0.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -20, 3.0e38], np.float32),
    ]).astype(np.float32)
    got = oracle.f32_to_bf16_n(v)
    ref = refmath.bf16_from_f32(v)
    np.testing.assert_array_equal(got, ref)


def test_f64_to_bf16_rounds_once():
    g = np.random.default_rng(2)
    d = g.standard_normal(200000) * 10.0 ** g.integers(-30, 30, 200000)
    # exact bf16 midpoints, and midpoints nudged by one binary64 ulp either way
    base = refmath.bf16_to_f32(g.integers(0x0080, 0x7F00, 5000).astype(np.uint16)).astype(np.float64)
    mids = base * (1 + 2.0 ** -8)
    d = np.concatenate([d, mids, np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf), -mids])
    got = oracle.f64_to_bf16_n(d)
    ref = refmath.bf16_from_f64(d)
    np.testing.assert_array_equal(got, ref)
    # a value just above a bf16 midpoint that binary32 rounding would pull onto it
    v = 1.0 + 2.0 ** -8 + 2.0 ** -40
    assert oracle.f64_to_bf16(v) == 0x3F81
    assert oracle.f64_to_bf16(1.0 + 2.0 ** -8) == 0x3F80  # tie -> even
    assert oracle.f64_to_bf16(1.0 + 3 * 2.0 ** -8) == 0x3F82  # tie -> even (up)


# ---------------------------------------------------------------- exp_ref, step by step
# The pinned definition of e^t (Cody & Waite 1980 reduction, degree-7 Taylor
# polynomial by Horner's rule with fused multiply-adds, scaling by 2^n), emulated
# here with exact rationals: each fp32 operation is its exact result rounded once
# (an fma rounds a*b + c once), constants are the nearest binary32 values of the
# mathematical constants.  A different polynomial degree, Horner order, a missing
# low part of ln 2 or an unfused step changes some of these bits.

def _emul_exp(t: float) -> float:
    F = Fraction
    log2e, ln2_hi = F(_rn32(LOG2E)), F(_rn32(LN2))
    ln2_lo = F(_rn32(LN2 - ln2_hi))
    c = [F(_rn32(F(1, math.factorial(m)))) for m in range(8)]
    t = F(t)
    n = refmath.rint_half_even(F(_rn32(t * log2e)))
    r = F(_rn32(-n * ln2_hi + t))
    r = F(_rn32(-n * ln2_lo + r))
    p = c[7]
    for m in range(6, -1, -1):
        p = F(_rn32(p * r + c[m]))
    return float(p * F(2) ** n)   # exact: the result stays in the normal range for |t| <= 80


def _emul_sigmoid(z: float) -> float:
    zc = min(max(z, -80.0), 80.0)
    e = Fraction(_emul_exp(-zc))
    return _rn32(Fraction(1) / Fraction(_rn32(1 + e)))


def _exp_points():
    g = np.random.default_rng(7)
    pts = np.concatenate([
        g.uniform(-80, 80, 160), g.uniform(-1, 1, 60), g.uniform(-1e-3, 1e-3, 20),
        np.array([0.0, 0.5, -0.5, 0.3465736, 0.3465737, 1.0, -1.0, 80.0, -80.0, 79.99, 44.3614, -44.3614]),
    ]).astype(np.float32)
    return pts


def test_exp_ref_matches_step_by_step_emulation():
    t = _exp_points()
    got = oracle.exp_ref_n(t)
    ref = np.array([_emul_exp(float(v)) for v in t], dtype=np.float32)
    np.testing.assert_array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_sigmoid_and_silu_match_step_by_step_emulation():
    z = np.concatenate([_exp_points(), np.array([-90.0, 95.0, -80.5], np.float32)]).astype(np.float32)
    s = oracle.sigmoid_ref_n(z)
    ref = np.array([_emul_sigmoid(float(v)) for v in z], dtype=np.float32)
    np.testing.assert_array_equal(s.view(np.uint32), ref.view(np.uint32))
    silu = oracle.silu_ref_n(z)
    ref_silu = np.array([_rn32(Fraction(float(v)) * Fraction(float(r))) for v, r in zip(z, ref)], dtype=np.float32)
    np.testing.assert_array_equal(silu.view(np.uint32), ref_silu.view(np.uint32))
