"""float8_e5m2 codec, written from the format's definition (oracle; tests only).

"Fp8 Quantization Support" (compressed-tensors PR 62), description: fp8 is
float8_e4m3fn for now, and float8_e5m2 is the named future extension of the
same quantization scheme.  Its bit layout is the OCP 8-bit floating point
"E5M2" encoding: 1 sign bit, 5 exponent bits with bias 15, 2 mantissa bits;
exponent field 0 holds subnormals m * 2^-16; exponent field 31 holds +-inf
(mantissa 0) and NaN (mantissa != 0).  The largest finite value is
1.75 * 2^15 = 57344.

``encode`` is the same saturating round-to-nearest-even cast as the e4m3
one: the nearest point of the finite grid, exact ties to the code with an
even mantissa, magnitudes above 57344 (and infinities) clamped to 57344, the
sign kept, NaN to a NaN code (0x7F with the sign).
"""
import numpy as np

E5M2_MAX = 57344.0
_MAX_CODE = 0x7B
_NAN_CODE = 0x7F


def decode(codes):
    """Exact value of each e5m2 byte, as float64 (+-inf and NaN included)."""
    b = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = b >> 7
    e = (b >> 2) & 0x1F
    m = b & 0x3
    mag = np.where(e == 0,
                   np.ldexp(m.astype(np.float64), -16),
                   np.ldexp(1.0 + m / 4.0, e - 15))
    mag = np.where(e == 31, np.where(m == 0, np.inf, np.nan), mag)
    return np.where(s == 1, -mag, mag)


def positive_grid():
    """The 124 non-negative finite values, indexed by their code 0x00..0x7B."""
    return decode(np.arange(_MAX_CODE + 1, dtype=np.uint8))


def encode(v):
    """Saturating RNE encoding of float32 values into e5m2 codes (uint8)."""
    v = np.asarray(v, dtype=np.float32)
    a = np.abs(v.astype(np.float64))
    sign = np.signbit(v).astype(np.uint8) << 7
    grid = positive_grid()
    finite = np.isfinite(a)
    a_f = np.where(finite, a, 0.0)
    lo = np.clip(np.searchsorted(grid, a_f, side="right") - 1, 0, _MAX_CODE)
    hi = np.minimum(lo + 1, _MAX_CODE)
    d_lo = a_f - grid[lo]
    d_hi = grid[hi] - a_f
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (lo % 2 == 1))
    code = np.where(take_hi, hi, lo)
    code = np.where(a_f >= E5M2_MAX, _MAX_CODE, code)      # saturate
    code = np.where(np.isinf(a), _MAX_CODE, code)
    code = np.where(np.isnan(a), _NAN_CODE, code)
    return (code.astype(np.uint8) | sign).astype(np.uint8)
