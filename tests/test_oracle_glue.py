"""Pins of the oracle's block glue (residual add, RMS normalization, gated
activation): closed forms, exact rational emulation, a library cast and
invariants -- facts fixed outside the oracle's own formulas."""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import oracle.glue
from oracle.w8a8 import bf16_bits_to_f32
from fp8_w8a8_quantized_amd import synth


def _bits_of(values_f32):
    return (np.asarray(values_f32, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _round_frac(x, mant_bits, min_exp):
    """Round a Fraction to the nearest binary value with mant_bits significant
    bits (ties to even), with a floor exponent for subnormals."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = math.floor(math.log2(a.numerator) - math.log2(a.denominator))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    step = Fraction(2) ** max(e - (mant_bits - 1), min_exp)
    q, r = divmod(a, step)
    if r * 2 > step or (r * 2 == step and q % 2 == 1):
        q += 1
    return sign * q * step


def _nearest_bf16_bits(x):
    v = _round_frac(Fraction(x), 8, -133)
    return int(_bits_of([float(v)])[0])


def test_f32_to_bf16_matches_torch_cast():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 20000),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.005859375, 65504.0, 3.0e38, 1e-40], np.float32)])
    x = x.astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.f32_to_bf16_bits(x), ref)


def test_f64_to_bf16_is_nearest_ties_even():
    rng = np.random.default_rng(1)
    xs = list(rng.standard_normal(300) * 10.0 ** rng.integers(-20, 20, 300))
    # exact ties between neighbouring bf16 values: 1 + 2^-8 (tie, even is 1), 1 + 3 * 2^-8 (tie, even is 1 + 2^-6)
    xs += [1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 2.0 ** -130 * 1.5]
    got = oracle.f64_to_bf16_bits(np.array(xs))
    for x, g in zip(xs, got):
        assert int(g) == _nearest_bf16_bits(x), x


def test_add_bf16_exact_rational_emulation():
    rng = np.random.default_rng(2)
    h = _bits_of(rng.standard_normal(2000).astype(np.float32) * 4)
    d = _bits_of((rng.standard_normal(2000) * 10.0 ** rng.integers(-8, 3, 2000)).astype(np.float32))
    got = oracle.add_bf16(h, d)
    hf, df = bf16_bits_to_f32(h), bf16_bits_to_f32(d)
    for i in range(len(h)):
        s32 = _round_frac(Fraction(float(hf[i])) + Fraction(float(df[i])), 24, -149)
        assert int(got[i]) == _nearest_bf16_bits(float(s32)), i


def test_add_bf16_closed_forms():
    one, two = _bits_of([1.0])[0], _bits_of([2.0])[0]
    assert oracle.add_bf16(np.array([one]), np.array([one]))[0] == two
    x = _bits_of([3.5, -7.25])
    assert np.all(bf16_bits_to_f32(oracle.add_bf16(x, x ^ np.uint16(0x8000))) == 0)


def test_rmsnorm_closed_forms():
    # a row of +-1: mean square 1, y = +-1/sqrt(1 + 1e-5) = +-0.999995 -> bf16 +-1
    row = _bits_of(np.where(np.arange(64) % 3 == 0, -1.0, 1.0))
    y = bf16_bits_to_f32(oracle.rmsnorm(row[None, :]))[0]
    assert np.array_equal(y, np.where(np.arange(64) % 3 == 0, -1.0, 1.0))
    # one-hot of height 8 in 64 columns: mean square 1, y0 = 8 / sqrt(1 + 1e-5) -> bf16 8
    oh = np.zeros(64, np.float32); oh[5] = 8.0
    y = bf16_bits_to_f32(oracle.rmsnorm(_bits_of(oh)[None, :]))[0]
    assert y[5] == 8.0 and np.count_nonzero(y) == 1
    # a constant small row where eps matters: y = c / sqrt(c^2 + 1e-5)
    c = float(bf16_bits_to_f32(_bits_of([0.01]))[0])
    y = oracle.rmsnorm(np.full((1, 32), _bits_of([0.01])[0]))
    assert int(y[0, 0]) == _nearest_bf16_bits(c / math.sqrt(c * c + 1e-5))


def test_rmsnorm_invariants():
    rng = np.random.default_rng(3)
    x = _bits_of(rng.standard_normal((5, 96)).astype(np.float32))
    y = oracle.rmsnorm(x)
    assert np.array_equal(oracle.rmsnorm(x ^ np.uint16(0x8000)), y ^ np.uint16(0x8000))   # odd function
    for r in range(5):                                                                     # rows independent
        assert np.array_equal(oracle.rmsnorm(x[r:r + 1]), y[r:r + 1])
    # the output's mean square is 1 up to eps and bf16 rounding
    yf = bf16_bits_to_f32(y).astype(np.float64)
    assert np.allclose(np.mean(yf * yf, axis=1), 1.0, atol=0.02)


def test_silu_mul_closed_forms():
    def one(g, u):
        gu = _bits_of([g, u])[None, :]
        return float(bf16_bits_to_f32(oracle.silu_mul(gu, 1))[0, 0])
    assert one(0.0, 5.0) == 0.0
    assert one(-100.0, 3.0) == 0.0
    assert one(32.0, 1.0) == 32.0                     # silu(g) = g (1 - e^-g + ...) -> bf16 32
    # silu(1) = e / (1 + e) (textbook value 0.7310585786...), times 1 and times 2
    assert _bits_of([one(1.0, 1.0)])[0] == _nearest_bf16_bits(math.e / (1 + math.e))
    assert _bits_of([one(1.0, 2.0)])[0] == _nearest_bf16_bits(2 * math.e / (1 + math.e))
    # the gate is the first half: swapping halves changes the result
    assert one(2.0, 1.0) != one(1.0, 2.0)


def test_silu_odd_part_identity():
    # silu(x) - silu(-x) = x exactly; after one bf16 rounding each side is within half a step
    xs = np.linspace(-6, 6, 97)
    xs = bf16_bits_to_f32(_bits_of(xs)).astype(np.float64)
    gu_p = _bits_of(np.stack([xs, np.ones_like(xs)], 1).reshape(-1))
    gu_n = _bits_of(np.stack([-xs, np.ones_like(xs)], 1).reshape(-1))
    p = bf16_bits_to_f32(oracle.silu_mul(gu_p.reshape(-1, 2), 1))[:, 0].astype(np.float64)
    n = bf16_bits_to_f32(oracle.silu_mul(gu_n.reshape(-1, 2), 1))[:, 0].astype(np.float64)
    tol = (np.abs(p) + np.abs(n)) * 2.0 ** -8 + 1e-30
    assert np.all(np.abs(p - n - xs) <= tol)


def test_ulp_distance():
    a = _bits_of([1.0, -1.0, 0.0])
    b = _bits_of([1.0078125, -1.0078125, -0.0])
    assert list(oracle.bf16_ulp_distance(a, b)) == [1, 1, 0]


def test_bf16_rounding_is_monotone_and_symmetric_so_row_max_commutes():
    """The statistics pass of the fused normalization takes a row's largest
    |y| = |bf16(h' * g)| as bf16(max |h'| * g): that holds because rounding to
    nearest is non-decreasing and odd.  Checked on sorted random doubles
    (including exact bf16 midpoints and their neighbours) and on rows."""
    rng = np.random.default_rng(12)
    mids = []
    for e in range(-20, 20):  # exact midpoints between consecutive bf16 values, and one ulp either side
        m = rng.integers(128, 256, 64).astype(np.float64)
        mid = (m + 0.5) * 2.0 ** (e - 7)
        mids += [mid, np.nextafter(mid, 0), np.nextafter(mid, np.inf)]
    x = np.sort(np.concatenate([rng.standard_normal(200000) * 10.0 ** rng.uniform(-6, 6, 200000)] + mids))
    r = oracle.bf16_bits_to_f32(oracle.glue.f64_to_bf16_bits(x)).astype(np.float64)
    assert np.all(np.diff(r) >= 0)
    neg = oracle.bf16_bits_to_f32(oracle.glue.f64_to_bf16_bits(-x)).astype(np.float64)
    assert np.array_equal(neg, -r)
    for _ in range(50):
        h = synth.activations(int(rng.integers(1, 1000)), 1, int(rng.integers(1, 5000)), outliers=True)
        hx = oracle.bf16_bits_to_f32(h).astype(np.float64)
        g = 1.0 / np.sqrt(np.mean(hx * hx) + 1e-5)
        ymax = np.max(oracle.glue.f64_to_bf16_bits(hx * g) & 0x7FFF)
        assert ymax == (oracle.glue.f64_to_bf16_bits(np.max(np.abs(hx)) * g) & 0x7FFF)
