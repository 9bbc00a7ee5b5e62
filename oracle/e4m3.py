"""float8_e4m3fn codec, written from the format's definition (oracle; tests only).

The pages name the dtype only ("Prototype FP8Linear W8A8 runtime quantization",
opening post; "Fp8 Quantization Support", description).  Its bit layout is the
OCP 8-bit floating point "E4M3" encoding in the finite-only ("fn") variant:
1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0
holds subnormals m * 2^-9; the single pattern S.1111.111 is NaN; there is no
infinity, so the largest finite value is 1.75 * 2^8 = 448.

``encode`` is the plain definition of a saturating round-to-nearest-even cast:
pick the nearest point of the finite e4m3 grid, break exact ties towards the
code with an even mantissa, clamp magnitudes above 448 to 448, keep the sign
(including the sign of zero), and send NaN to the NaN code.
"""
import numpy as np

E4M3_MAX = 448.0
_NAN_CODE = 0x7F


def decode(codes):
    """Exact value of each e4m3fn byte, as float64 (NaN for 0x7F/0xFF)."""
    b = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = b >> 7
    e = (b >> 3) & 0xF
    m = b & 0x7
    mag = np.where(e == 0,
                   np.ldexp(m.astype(np.float64), -9),
                   np.ldexp(1.0 + m / 8.0, e - 7))
    val = np.where(s == 1, -mag, mag)
    return np.where((e == 15) & (m == 7), np.nan, val)


def positive_grid():
    """The 127 non-negative finite values, indexed by their code 0x00..0x7E."""
    return decode(np.arange(0x7F, dtype=np.uint8))


def encode(v):
    """Saturating RNE encoding of float32 values into e4m3fn codes (uint8).

    The input is widened to float64, which is exact for float32, so every
    distance below is computed exactly (both neighbours are within a factor of
    two of the value, or the lower one is zero).
    """
    v = np.asarray(v, dtype=np.float32)
    a = np.abs(v.astype(np.float64))
    sign = np.signbit(v).astype(np.uint8) << 7
    grid = positive_grid()
    finite = np.isfinite(a)
    a_f = np.where(finite, a, 0.0)
    # index of the largest grid point <= a (0 .. 126)
    lo = np.clip(np.searchsorted(grid, a_f, side="right") - 1, 0, 126)
    hi = np.minimum(lo + 1, 126)
    d_lo = a_f - grid[lo]
    d_hi = grid[hi] - a_f
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (lo % 2 == 1))
    code = np.where(take_hi, hi, lo)
    code = np.where(a_f >= E4M3_MAX, 126, code)            # saturate
    code = np.where(np.isinf(a), 126, code)                # +-inf saturates too
    code = np.where(np.isnan(a), _NAN_CODE, code)
    return (code.astype(np.uint8) | sign).astype(np.uint8)
