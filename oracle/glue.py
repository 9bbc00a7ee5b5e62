"""Steps that feed the linears of a Llama-shaped decoder block (oracle; tests only).

The pages describe the linear layer alone.  The chained-linears workload (a
32-layer decoder-shaped stack) also needs what sits between the linears, and
the pages fix none of it, so each definition below is a reading:
  * residual add in the residual stream's precision: both bf16 operands are
    added in float32 (one rounding) and the sum is rounded to bf16;
  * RMS normalization with unit weight: y = x / sqrt(mean(x^2) + eps),
    eps = 1e-5, rounded once to bf16;
  * gated activation (gate half first): y = silu(g) * u with
    silu(g) = g / (1 + exp(-g)), rounded once to bf16.
The review of "[WIP] FP8 support" (text-generation-inference PR 1484) asks to
remove the unnecessary operations around the FP8 GEMM; the HIP side therefore
fuses these producers with the activation quantization.  Here they are
computed unfused, from their plain definitions, in float64 (the add in
float32, as defined above) with a single rounding to bf16.
"""
import numpy as np

from .w8a8 import bf16_bits_to_f32, to_bf16_rne


def f64_to_bf16_bits(x):
    """float64 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    r = to_bf16_rne(np.asarray(x, dtype=np.float64))
    # every bf16 value is a float32 value: the conversion below is exact
    return (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def f32_to_bf16_bits(x):
    """float32 -> bf16 bit patterns, round to nearest even (NaN stays NaN)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = ((u & 0x7FFFFFFF) > 0x7F800000)
    return np.where(nan, ((u >> 16) | 0x40).astype(np.uint16), rounded)


def add_bf16(h_bits, d_bits):
    """Residual add: bf16(fl32(h + d)) as bf16 bits."""
    h = bf16_bits_to_f32(h_bits)
    d = bf16_bits_to_f32(d_bits)
    with np.errstate(over="ignore", invalid="ignore"):
        s = (h + d).astype(np.float32)
    return f32_to_bf16_bits(s)


def rmsnorm(h_bits, eps=1e-5):
    """Unit-weight RMS normalization of each row, float64, rounded once to bf16."""
    x = bf16_bits_to_f32(h_bits).astype(np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return f64_to_bf16_bits(x / np.sqrt(ms + eps))


def silu_mul(gu_bits, cols):
    """silu(gate) * up for rows laid out [gate (cols) | up (cols)]; bf16 bits."""
    gu = bf16_bits_to_f32(gu_bits).astype(np.float64)
    g, u = gu[..., :cols], gu[..., cols:2 * cols]
    with np.errstate(over="ignore"):
        y = g / (1.0 + np.exp(-g)) * u
    return f64_to_bf16_bits(y)


def bf16_ulp_distance(a_bits, b_bits):
    """Distance in bf16 steps between two arrays of (finite) bf16 bit patterns."""
    def ordered(b):
        b = np.asarray(b, dtype=np.uint16).astype(np.int64)
        return np.where(b & 0x8000, -(b & 0x7FFF), b)
    return np.abs(ordered(a_bits) - ordered(b_bits))
