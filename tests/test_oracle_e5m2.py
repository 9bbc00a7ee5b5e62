"""Pins of the oracle's e5m2 codec and of the format parameter of the
quantization and GEMM steps: the closed-form decode, the 256-pattern table of
a library dtype, an exhaustive brute force over bf16, the library cast, and
exact integer arithmetic."""
from fractions import Fraction

import numpy as np
import torch

import oracle
from oracle import e5m2

ALL_BYTES = np.arange(256, dtype=np.uint8)
ALL_BF16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)


def test_e5m2_decode_spot_values():
    d = e5m2.decode(np.array([0x7B, 0x01, 0x04, 0x3C, 0x00, 0x3D, 0xFB, 0x03], np.uint8))
    assert d.tolist() == [57344.0, 2.0 ** -16, 2.0 ** -14, 1.0, 0.0, 1.25, -57344.0, 3 * 2.0 ** -16]
    assert np.isinf(e5m2.decode(np.array([0x7C, 0xFC], np.uint8))).all()
    assert np.isnan(e5m2.decode(np.array([0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF], np.uint8))).all()
    z = e5m2.decode(np.array([0x80], np.uint8))[0]
    assert z == 0.0 and np.signbit(z)


def test_e5m2_decode_table_matches_torch():
    ours = e5m2.decode(ALL_BYTES)
    theirs = torch.from_numpy(ALL_BYTES.copy()).view(torch.float8_e5m2).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(theirs))
    ok = ~np.isnan(ours)
    assert np.array_equal(ours[ok], theirs[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(theirs[ok]))


def test_e5m2_round_trip():
    vals = e5m2.decode(ALL_BYTES)
    finite = np.isfinite(vals)
    assert np.array_equal(e5m2.encode(vals[finite].astype(np.float32)), ALL_BYTES[finite])
    assert np.all(e5m2.encode(np.array([np.inf, -np.inf], np.float32)) == np.array([0x7B, 0xFB], np.uint8))
    assert np.all((e5m2.encode(np.array([np.nan], np.float32)) & 0x7F) == 0x7F)


def test_e5m2_exhaustive_bf16_brute_force():
    x = oracle.bf16_bits_to_f32(ALL_BF16)
    fin = np.isfinite(x)
    xv = x[fin].astype(np.float64)
    grid = e5m2.positive_grid()                      # 124 values
    a = np.abs(xv)
    dist = np.abs(a[:, None] - grid[None, :])
    best = dist.min(axis=1, keepdims=True)
    cand = dist == best                              # one or two nearest points
    codes = np.arange(len(grid))
    # ties go to the even code (even mantissa); beyond the largest value: saturate
    pick = np.where(cand.sum(1) == 2, np.where(cand & (codes[None, :] % 2 == 0), codes[None, :], 999).min(1),
                    np.argmax(cand, axis=1))
    pick = np.where(a >= 57344.0, 0x7B, pick)
    ref = (pick.astype(np.uint8) | (np.signbit(xv).astype(np.uint8) << 7)).astype(np.uint8)
    assert np.array_equal(e5m2.encode(x[fin]), ref)


def test_e5m2_matches_torch_cast_after_clamp():
    rng = np.random.default_rng(11)
    v = (rng.standard_normal(200000) * 10.0 ** rng.integers(-8, 6, 200000)).astype(np.float32)
    v = np.concatenate([v, np.array([57344.0, 61440.0, 61439.0, -70000.0, 2.0 ** -17, 3 * 2.0 ** -18], np.float32)])
    clamped = torch.from_numpy(np.clip(v, -57344.0, 57344.0))
    theirs = clamped.to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert np.array_equal(e5m2.encode(v), theirs)


def test_quant_with_e5m2_scale_and_extremes():
    rng = np.random.default_rng(12)
    x = oracle.f32_to_bf16_bits(rng.standard_normal((7, 33)).astype(np.float32) * 3)
    q, s = oracle.quant_dynamic(x, "e5m2")
    xf = oracle.bf16_bits_to_f32(x)
    assert s == np.float32(np.max(np.abs(xf)) / np.float32(57344.0))
    i = np.unravel_index(np.argmax(np.abs(xf)), xf.shape)
    assert q[i] & 0x7F == 0x7B
    assert np.array_equal(oracle.quant_dynamic(x ^ np.uint16(0x8000), "e5m2")[0], q ^ np.uint8(0x80))


def test_gemm_mixed_formats_exact_on_small_shapes():
    rng = np.random.default_rng(13)
    for fa, fw in (("e5m2", "e5m2"), ("e4m3", "e5m2"), ("e5m2", "e4m3")):
        a = rng.integers(0, 256, (3, 9)).astype(np.uint8)
        w = rng.integers(0, 256, (4, 9)).astype(np.uint8)
        da, dw = oracle.FORMATS[fa][0](a), oracle.FORMATS[fw][0](w)
        a[~np.isfinite(da)] = 0
        w[~np.isfinite(dw)] = 0
        da, dw = oracle.FORMATS[fa][0](a), oracle.FORMATS[fw][0](w)
        got = oracle.gemm_exact(a, w, fa, fw)
        for m in range(3):
            for n in range(4):
                exact = sum(Fraction(float(da[m, k])) * Fraction(float(dw[n, k])) for k in range(9))
                assert abs(Fraction(float(got[m, n])) - exact) <= abs(exact) * Fraction(1, 2 ** 50)
