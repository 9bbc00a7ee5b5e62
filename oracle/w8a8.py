"""W8A8 FP8 linear layer, step by step on the CPU (oracle; tests only).

The method, from the pages:
  * "Prototype FP8Linear W8A8 runtime quantization", opening post: both the
    weights and the activations are quantized to float8_e4m3fn at run time and
    an FP8 W8A8 GEMM multiplies them.
  * "Fp8 Quantization Support", description and recipe: symmetric (no zero
    point) float quantization, one scale per tensor for weights and input
    activations; a float format's range and rounding differ from int8's.
  * "[Kernel] Implement fallback for FP8 channelwise using torch._scaled_mm",
    description: channelwise weights (one scale per output channel) are
    served by a per-tensor scaled GEMM followed by a rescale of each output
    column.

Readings where the pages are silent: the dynamic scale is amax/448 rounded
once to float32 (448 being the largest finite e4m3fn value), with
amax == 0 mapping to scale 1.0; values are divided (not multiplied by a
reciprocal) in float32; the cast saturates and rounds to nearest even; the
weight has nn.Linear layout [N, K] and output channel n is weight row n; an
optional bias is added after scaling.

Precision: the quantization steps are float32, as the GPU computes them, so
that both sides take every rounding decision in the same precision.  The GEMM
is exact (fp64 of decoded e4m3 values is exact for K < 171,196; int64 is exact
always), and the epilogue is fp64 and left unrounded.
"""
import numpy as np

from . import e4m3, e5m2
from .e4m3 import E4M3_MAX, decode, encode

_F32_MAX = np.float32(E4M3_MAX)

# The two fp8 formats: (decode, encode, largest finite value).  e4m3 is the
# pages' format; e5m2 is the extension "Fp8 Quantization Support" names.
FORMATS = {"e4m3": (e4m3.decode, e4m3.encode, np.float32(e4m3.E4M3_MAX)),
           "e5m2": (e5m2.decode, e5m2.encode, np.float32(e5m2.E5M2_MAX))}


def bf16_bits_to_f32(bits):
    """bf16 bit patterns (uint16) -> float32; exact (the bits move up 16)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def amax(x_f32):
    """max |x| over the whole array as float32 (0 for an empty array)."""
    x_f32 = np.asarray(x_f32, dtype=np.float32)
    if x_f32.size == 0:
        return np.float32(0.0)
    return np.float32(np.max(np.abs(x_f32)))


def scale_from_amax(a, fmt="e4m3"):
    """Per-tensor scale mapping amax onto the format's largest value.

    s = fl32(amax / max) (one correctly rounded float32 division; max = 448
    for e4m3, 57344 for e5m2); an all-zero (or empty) tensor has no range to
    map and takes s = 1.
    """
    a = np.float32(a)
    if a == 0:
        return np.float32(1.0)
    return np.float32(a / FORMATS[fmt][2])


def quant_static(x_bits, scale, fmt="e4m3"):
    """Quantize bf16 bits with a given float32 scale: enc(fl32(x / scale)).

    The division is float32 and correctly rounded, then the saturating RNE
    encoder of the format runs on that float32 quotient.
    """
    x = bf16_bits_to_f32(x_bits)
    s = np.float32(scale)
    with np.errstate(over="ignore", divide="ignore", invalid="ignore"):
        v = (x / s).astype(np.float32)
    return FORMATS[fmt][1](v)


def quant_dynamic(x_bits, fmt="e4m3"):
    """Dynamic per-tensor activation quantization: returns (codes, scale)."""
    x = bf16_bits_to_f32(x_bits)
    s = scale_from_amax(amax(x), fmt)
    return quant_static(x_bits, s, fmt), s


def quant_weight(w_bits, per_channel, fmt="e4m3"):
    """Weight quantization, [N, K] bf16 bits -> (codes [N, K], scales).

    Per tensor: one scale from the amax of the whole matrix (shape [1]).
    Per channel: row n (output channel n) gets its own scale from its own
    amax (shape [N]); an all-zero row gets scale 1.
    """
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    if not per_channel:
        q, s = quant_dynamic(w_bits, fmt)
        return q, np.array([s], dtype=np.float32)
    w = bf16_bits_to_f32(w_bits)
    a = (np.max(np.abs(w), axis=1) if w.shape[1] else np.zeros(w.shape[0])).astype(np.float32)
    # the per-tensor rule applied to each row: fl32(amax_n / max), 1 when 0
    s = np.where(a == 0, np.float32(1.0), a / FORMATS[fmt][2]).astype(np.float32)
    with np.errstate(over="ignore", divide="ignore", invalid="ignore"):
        v = (w / s[:, None]).astype(np.float32)
    return FORMATS[fmt][1](v), s


def gemm_exact(a_q, w_q, fmt_a="e4m3", fmt_w="e4m3"):
    """acc[m, n] = sum_k dec(A_q[m, k]) * dec(W_q[n, k]).

    e4m3 x e4m3: every decoded value times 512 is an integer, so each
    product is an integer multiple of 2^-18 below 448^2 and the float64 sum
    of K of them is exact while K * 448^2 * 2^18 < 2^53, i.e. K < 171,196.
    With an e5m2 operand (values are multiples of 2^-16 up to 57344) the
    products span more than 53 bits, so the float64 sum may round: its error
    is at most K * 2^-53 * sum_k |a_k w_k|, ten orders below the parity
    tolerance.
    """
    a_q = np.asarray(a_q, dtype=np.uint8)
    w_q = np.asarray(w_q, dtype=np.uint8)
    k = a_q.shape[1]
    if fmt_a == "e4m3" and fmt_w == "e4m3" and k >= 171196:
        raise ValueError("K too large for the exact float64 path")
    return FORMATS[fmt_a][0](a_q) @ FORMATS[fmt_w][0](w_q).T


def scaled_mm(a_q, w_q, s_a, s_w, per_channel, bias_bits=None, acc=None, fmt_a="e4m3", fmt_w="e4m3"):
    """The rescale epilogue in float64, unrounded.

    out[m, n] = acc[m, n] * s_a * s_w[n] (+ bias[n]); per tensor uses s_w[0]
    for every column.  Because s_w[n] does not vary along k, this equals a
    per-tensor scaled GEMM followed by a rescale of column n.
    """
    if acc is None:
        acc = gemm_exact(a_q, w_q, fmt_a, fmt_w)
    s_w = np.asarray(s_w, dtype=np.float32).astype(np.float64)
    col = s_w if per_channel else np.full(acc.shape[1], s_w[0])
    out = acc * np.float64(np.float32(s_a)) * col[None, :]
    if bias_bits is not None:
        out = out + bf16_bits_to_f32(bias_bits).astype(np.float64)[None, :]
    return out


def dequant_row_norms(q, scales, per_row, fmt="e4m3"):
    """L2 norm of each dequantized row: ||dec(q[r, :]) * scale_r||_2 (fp64)."""
    d = FORMATS[fmt][0](np.asarray(q, dtype=np.uint8))
    s = np.asarray(scales, dtype=np.float32).astype(np.float64)
    s = s if per_row else np.full(d.shape[0], s.reshape(-1)[0])
    return np.sqrt(np.sum(d * d, axis=1)) * np.abs(s)


def to_bf16_rne(x):
    """Round float64 values to the nearest bfloat16 (ties to even); float64.

    bfloat16 keeps 8 significant bits; below 2^-126 its step is 2^-133.
    Used only to report what an ideal bf16 output would be.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                       # x = m * 2^e, 0.5 <= |m| < 1
    q = np.ldexp(1.0, np.maximum(e - 8, -133))
    r = np.rint(x / q) * q                    # x / q is exact (power of two)
    return np.where(x == 0, x, r)
