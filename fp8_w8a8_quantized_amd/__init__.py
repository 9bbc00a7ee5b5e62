"""MI355X-native FP8 W8A8 linear layer (gfx950 HIP kernels behind a C ABI).

The compute path lives in ``libfp8w8a8.so`` (built from ``csrc/``, declared
in ``include/fp8w8a8.h``).  This module only marshals torch device tensors
and the current HIP stream into those C calls: every step of the layer runs
in the library's kernels.  Importing the package does not load the library;
the first call does, and raises if it is missing -- there is no CPU path.

e4m3fn tensors are torch.uint8 holding the codes; bf16 tensors are
torch.bfloat16; scales are float32 device tensors.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp8w8a8.so")

FP8_SCALE_PER_TENSOR = 0
FP8_SCALE_PER_CHANNEL = 1
FP8_ACCUM_FP32 = 0
FP8_ACCUM_FP8_MFMA = 1
ACCUM = {"fp32": FP8_ACCUM_FP32, "fp8": FP8_ACCUM_FP8_MFMA}
E4M3_MAX = 448.0

# name -> (restype, argtypes); mirrors include/fp8w8a8.h
_P, _I64, _I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
SIGNATURES = {
    "fp8_quant_workspace_bytes": (ctypes.c_size_t, []),
    "fp8_last_error": (ctypes.c_char_p, []),
    "fp8_quant_dynamic": (_I, [_P, _I64, _I64, _I64, _P, _I64, _P, _P, _P]),
    "fp8_quant_static": (_I, [_P, _I64, _I64, _I64, _P, _P, _I64, _P]),
    "fp8_quant_dynamic_per_row": (_I, [_P, _I64, _I64, _I64, _P, _I64, _P, _P]),
    "fp8_scaled_mm": (_I, [_P, _I64, _P, _I64, _P, _P, _I, _P, _P, _I64, _I64, _I64, _I64, _P]),
    "fp8_quant_dynamic_fmt": (_I, [_P, _I64, _I64, _I64, _I, _P, _I64, _P, _P, _P]),
    "fp8_quant_static_fmt": (_I, [_P, _I64, _I64, _I64, _I, _P, _P, _I64, _P]),
    "fp8_quant_dynamic_per_row_fmt": (_I, [_P, _I64, _I64, _I64, _I, _P, _I64, _P, _P]),
    "fp8_scaled_mm_fmt": (_I, [_P, _I64, _I, _P, _I64, _I, _P, _P, _I, _I, _P, _P, _I64, _I64, _I64, _I64, _P]),
    "fp8_norm_quant_workspace_bytes": (ctypes.c_size_t, [_I64]),
    "fp8_add_rmsnorm_quant_dynamic": (_I, [_P, _I64, _P, _I64, _P, _I64, _I64, _I64, ctypes.c_float,
                                           _P, _I64, _P, _I64, _P, _P, _P]),
    "fp8_silu_mul_quant_dynamic": (_I, [_P, _I64, _I64, _I64, _P, _I64, _P, _I64, _P, _P, _P]),
    "fp8_linear_workspace_bytes": (ctypes.c_size_t, []),
    "fp8_linear_dynamic": (_I, [_P, _I64, _P, _I64, _P, _I, _I, _P, _P, _I64, _P, _P, _I64, _I64, _I64, _I64,
                                _P, _P]),
    "fp8_linear_dynamic_noalloc": (_I, [_P, _I64, _P, _I64, _P, _I, _I, _P, _P, _I64, _P, _P, _I64, _I64, _I64,
                                        _I64, _P]),
}

_lib = None


class Fp8Error(RuntimeError):
    pass


def lib():
    """The loaded C library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise Fp8Error(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                           "(python -m fp8_w8a8_quantized_amd._build); there is no fallback path")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(status, fn):
    if status != 0:
        msg = lib().fp8_last_error().decode(errors="replace")
        raise Fp8Error(f"{fn} returned status {status}: {msg}")


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


# ---------------------------------------------------------------- validation
# Every tensor is checked (device, dtype, shape or element count, strides)
# before any library call: the kernels trust the sizes they are given, so a
# short scale vector or a host tensor would otherwise become an out-of-range
# device access.

def _on_gpu(t):
    return t.is_cuda


def _device(t, name, device):
    if not _on_gpu(t):
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _mat(t, name, dtype, shape=None, device=None):
    """A 2-D tensor of `dtype` with unit column stride (any row pitch >= cols)."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a tensor")
    _device(t, name, device)
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != 2 or (t.size(1) > 1 and t.stride(1) != 1) or t.stride(0) < max(t.size(1), 1):
        raise ValueError(f"{name} must be 2-D with unit column stride and row pitch >= its columns")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _vec(t, name, dtype, n, device):
    """A contiguous tensor of exactly n elements of `dtype` on `device`."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a tensor")
    _device(t, name, device)
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.numel() != n:
        raise ValueError(f"{name} must have {n} element(s), got {t.numel()}")
    if n > 1 and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _workspace(t, name, nbytes, device):
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a tensor")
    _device(t, name, device)
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes, needs {nbytes}")
    return t


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def workspace_bytes():
    return int(lib().fp8_quant_workspace_bytes())


def new_workspace(device=None):
    return torch.empty(workspace_bytes(), dtype=torch.uint8, device=device or "cuda")


FORMAT = {"e4m3": 0, "e5m2": 1}


def _fmt(fmt):
    if fmt not in FORMAT:
        raise ValueError(f"unknown fp8 format {fmt!r} (expected one of {sorted(FORMAT)})")
    return FORMAT[fmt]


def _accum(accum):
    if accum not in ACCUM:
        raise ValueError(f"unknown accumulation mode {accum!r} (expected one of {sorted(ACCUM)})")
    return ACCUM[accum]


def quant_dynamic(x, workspace=None, q=None, scale=None, fmt="e4m3"):
    """Dynamic per-tensor quantization of bf16 x [rows, cols] into fmt codes.

    Returns (q uint8 [rows, cols], scale float32 [1]); the scale stays on the
    device.
    """
    _mat(x, "x", torch.bfloat16)
    dev = x.device
    rows, cols = x.shape
    f = _fmt(fmt)
    q = torch.empty((rows, cols), dtype=torch.uint8, device=dev) if q is None else q
    scale = torch.empty(1, dtype=torch.float32, device=dev) if scale is None else scale
    _mat(q, "q", torch.uint8, (rows, cols), dev)
    _vec(scale, "scale", torch.float32, 1, dev)
    workspace = new_workspace(dev) if workspace is None else workspace
    _workspace(workspace, "workspace", workspace_bytes(), dev)
    _check(lib().fp8_quant_dynamic_fmt(_ptr(x), rows, cols, x.stride(0), f, _ptr(q), q.stride(0),
                                       _ptr(scale), _ptr(workspace), _stream()), "fp8_quant_dynamic")
    return q, scale


def quant_static(x, scale, q=None, fmt="e4m3"):
    """Quantize bf16 x with a given device float32 scale; returns q uint8."""
    _mat(x, "x", torch.bfloat16)
    dev = x.device
    rows, cols = x.shape
    f = _fmt(fmt)
    _vec(scale, "scale", torch.float32, 1, dev)
    q = torch.empty((rows, cols), dtype=torch.uint8, device=dev) if q is None else q
    _mat(q, "q", torch.uint8, (rows, cols), dev)
    _check(lib().fp8_quant_static_fmt(_ptr(x), rows, cols, x.stride(0), f, _ptr(scale), _ptr(q),
                                      q.stride(0), _stream()), "fp8_quant_static")
    return q


def quant_dynamic_per_row(x, q=None, scales=None, fmt="e4m3"):
    """One scale per row (channelwise weight quantization): (q, scales [rows])."""
    _mat(x, "x", torch.bfloat16)
    dev = x.device
    rows, cols = x.shape
    f = _fmt(fmt)
    q = torch.empty((rows, cols), dtype=torch.uint8, device=dev) if q is None else q
    scales = torch.empty(rows, dtype=torch.float32, device=dev) if scales is None else scales
    _mat(q, "q", torch.uint8, (rows, cols), dev)
    _vec(scales, "scales", torch.float32, rows, dev)
    _check(lib().fp8_quant_dynamic_per_row_fmt(_ptr(x), rows, cols, x.stride(0), f, _ptr(q), q.stride(0),
                                               _ptr(scales), _stream()), "fp8_quant_dynamic_per_row")
    return q, scales


def quant_weight(w, per_channel, fmt="e4m3"):
    """Load-time weight quantization on the device: (w_q, s_w)."""
    if per_channel:
        return quant_dynamic_per_row(w, fmt=fmt)
    return quant_dynamic(w, fmt=fmt)


def _gemm_operands(a_q, w_q, s_a, s_w, per_channel, bias, out):
    """Validate the scaled GEMM's tensors; returns (M, N, K, out)."""
    _mat(a_q, "a_q", torch.uint8)
    dev = a_q.device
    _mat(w_q, "w_q", torch.uint8, device=dev)
    M, K = a_q.shape
    N, K2 = w_q.shape
    if K != K2:
        raise ValueError(f"K mismatch: a_q has {K}, w_q has {K2}")
    _vec(s_a, "s_a", torch.float32, 1, dev)
    _vec(s_w, "s_w", torch.float32, N if per_channel else 1, dev)
    if bias is not None:
        _vec(bias, "bias", torch.bfloat16, N, dev)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev) if out is None else out
    _mat(out, "out", torch.bfloat16, (M, N), dev)
    return M, N, K, out


def scaled_mm(a_q, w_q, s_a, s_w, per_channel, bias=None, out=None, accum="fp32", fmt_a="e4m3", fmt_w="e4m3"):
    """out[M, N] = bf16((A_q @ W_q^T) * s_a * s_w (+ bias)); W_q is [N, K].

    accum: "fp32" (fp32-class sums, default) or "fp8" (fp8 matrix cores for
    M > 64: twice the rate, 13-bit sums inside each group of 8 products).
    fmt_a / fmt_w: "e4m3" or "e5m2" codes.  The default (e4m3 codes, fp32
    sums) is the library's fp8_scaled_mm; other choices go through
    fp8_scaled_mm_fmt.
    """
    fa, fw, acc = _fmt(fmt_a), _fmt(fmt_w), _accum(accum)
    M, N, K, out = _gemm_operands(a_q, w_q, s_a, s_w, per_channel, bias, out)
    mode = FP8_SCALE_PER_CHANNEL if per_channel else FP8_SCALE_PER_TENSOR
    if fa == 0 and fw == 0 and acc == FP8_ACCUM_FP32:
        _check(lib().fp8_scaled_mm(_ptr(a_q), a_q.stride(0), _ptr(w_q), w_q.stride(0), _ptr(s_a), _ptr(s_w), mode,
                                   _ptr(bias), _ptr(out), out.stride(0), M, N, K, _stream()), "fp8_scaled_mm")
    else:
        _check(lib().fp8_scaled_mm_fmt(_ptr(a_q), a_q.stride(0), fa, _ptr(w_q), w_q.stride(0), fw, _ptr(s_a),
                                       _ptr(s_w), mode, acc, _ptr(bias), _ptr(out), out.stride(0), M, N, K,
                                       _stream()), "fp8_scaled_mm_fmt")
    return out


def linear_workspace_bytes():
    return int(lib().fp8_linear_workspace_bytes())


def new_linear_workspace(device=None):
    """Scratch workspace of linear_dynamic (no initialization needed)."""
    return torch.empty(linear_workspace_bytes(), dtype=torch.uint8, device=device or "cuda")


def linear_dynamic(x, w_q, s_w, per_channel, bias=None, workspace=None, a_q=None, s_a=None, out=None,
                   accum="fp32"):
    """The whole e4m3 W8A8 linear in one library call: dynamic per-tensor
    quantization of bf16 x [M, K] (codes a_q, scale s_a), then the scaled
    GEMM against w_q [N, K].

    Returns (out [M, N] bf16, a_q [M, K] uint8, s_a [1] float32).
    """
    acc = _accum(accum)
    _mat(x, "x", torch.bfloat16)
    dev = x.device
    M, K = x.shape
    a_q = torch.empty((M, K), dtype=torch.uint8, device=dev) if a_q is None else a_q
    s_a = torch.empty(1, dtype=torch.float32, device=dev) if s_a is None else s_a
    _mat(a_q, "a_q", torch.uint8, (M, K), dev)
    M, N, K, out = _gemm_operands(a_q, w_q, s_a, s_w, per_channel, bias, out)
    workspace = new_linear_workspace(dev) if workspace is None else workspace
    _workspace(workspace, "workspace", linear_workspace_bytes(), dev)
    mode = FP8_SCALE_PER_CHANNEL if per_channel else FP8_SCALE_PER_TENSOR
    _check(lib().fp8_linear_dynamic(_ptr(x), x.stride(0), _ptr(w_q), w_q.stride(0), _ptr(s_w), mode, acc,
                                    _ptr(bias), _ptr(a_q), a_q.stride(0), _ptr(s_a), _ptr(out), out.stride(0),
                                    M, N, K, _ptr(workspace), _stream()),
           "fp8_linear_dynamic")
    return out, a_q, s_a


def linear_dynamic_noalloc(x, w_q, s_w, per_channel, bias, a_q, s_a, out, accum="fp32"):
    """linear_dynamic for callers that cannot allocate: every output is the
    caller's, and the quantization's scratch is the library's own per-device
    array (calls that overlap on one device race).  Returns out."""
    acc = _accum(accum)
    _mat(x, "x", torch.bfloat16)
    dev = x.device
    M, K = x.shape
    _mat(a_q, "a_q", torch.uint8, (M, K), dev)
    M, N, K, out = _gemm_operands(a_q, w_q, s_a, s_w, per_channel, bias, out)
    mode = FP8_SCALE_PER_CHANNEL if per_channel else FP8_SCALE_PER_TENSOR
    _check(lib().fp8_linear_dynamic_noalloc(_ptr(x), x.stride(0), _ptr(w_q), w_q.stride(0), _ptr(s_w), mode, acc,
                                            _ptr(bias), _ptr(a_q), a_q.stride(0), _ptr(s_a), _ptr(out),
                                            out.stride(0), M, N, K, _stream()),
           "fp8_linear_dynamic_noalloc")
    return out


def linear(x, w_q, s_w, per_channel, bias=None, workspace=None, accum="fp32", fmt_a="e4m3", fmt_w="e4m3"):
    """The W8A8 linear: dynamic activation quantization then scaled GEMM.

    e4m3 codes on both sides go through linear_dynamic (one library call);
    other formats make the two calls.  workspace: a new_workspace() (or a
    new_linear_workspace(), the same size).
    """
    if fmt_a == "e4m3" and fmt_w == "e4m3":
        return linear_dynamic(x, w_q, s_w, per_channel, bias, workspace=workspace, accum=accum)[0]
    a_q, s_a = quant_dynamic(x, workspace=workspace, fmt=fmt_a)
    return scaled_mm(a_q, w_q, s_a, s_w, per_channel, bias, accum=accum, fmt_a=fmt_a, fmt_w=fmt_w)


def norm_workspace(rows, device=None):
    return torch.empty(int(lib().fp8_norm_quant_workspace_bytes(rows)), dtype=torch.uint8,
                       device=device or "cuda")


def add_rmsnorm_quant(h, delta=None, h_out=None, eps=1e-5, y_out=None, q=None, scale=None, workspace=None):
    """Residual add (optional), unit-weight RMS normalization and dynamic
    per-tensor quantization in one pass over h.

    Returns (q uint8, scale float32 [1], h_out or None, y_out or None):
    h_out receives bf16(h + delta) when delta is given; y_out, when given,
    receives the normalized bf16 values that were quantized.
    """
    _mat(h, "h", torch.bfloat16)
    dev = h.device
    rows, cols = h.shape
    if delta is not None:
        _mat(delta, "delta", torch.bfloat16, (rows, cols), dev)
        h_out = torch.empty_like(h) if h_out is None else h_out
        _mat(h_out, "h_out", torch.bfloat16, (rows, cols), dev)
    if y_out is not None:
        _mat(y_out, "y_out", torch.bfloat16, (rows, cols), dev)
    q = torch.empty((rows, cols), dtype=torch.uint8, device=dev) if q is None else q
    scale = torch.empty(1, dtype=torch.float32, device=dev) if scale is None else scale
    _mat(q, "q", torch.uint8, (rows, cols), dev)
    _vec(scale, "scale", torch.float32, 1, dev)
    workspace = norm_workspace(rows, dev) if workspace is None else workspace
    _workspace(workspace, "workspace", int(lib().fp8_norm_quant_workspace_bytes(rows)), dev)
    _check(lib().fp8_add_rmsnorm_quant_dynamic(
        _ptr(h), h.stride(0), _ptr(delta), delta.stride(0) if delta is not None else 0,
        _ptr(h_out if delta is not None else None), h_out.stride(0) if delta is not None else 0,
        rows, cols, ctypes.c_float(eps), _ptr(y_out), y_out.stride(0) if y_out is not None else 0,
        _ptr(q), q.stride(0), _ptr(scale), _ptr(workspace), _stream()), "fp8_add_rmsnorm_quant_dynamic")
    return q, scale, (h_out if delta is not None else None), y_out


def silu_mul_quant(gu, y_out=None, q=None, scale=None, workspace=None):
    """silu(gate) * up of a fused gate_up output [rows, 2 cols] (gate first),
    quantized with a dynamic per-tensor scale.  Returns (q, scale, y_out)."""
    _mat(gu, "gu", torch.bfloat16)
    dev = gu.device
    rows, two_cols = gu.shape
    if two_cols % 2:
        raise ValueError("gu must have an even number of columns (gate | up)")
    cols = two_cols // 2
    if y_out is not None:
        _mat(y_out, "y_out", torch.bfloat16, (rows, cols), dev)
    q = torch.empty((rows, cols), dtype=torch.uint8, device=dev) if q is None else q
    scale = torch.empty(1, dtype=torch.float32, device=dev) if scale is None else scale
    _mat(q, "q", torch.uint8, (rows, cols), dev)
    _vec(scale, "scale", torch.float32, 1, dev)
    workspace = new_workspace(dev) if workspace is None else workspace
    _workspace(workspace, "workspace", workspace_bytes(), dev)
    _check(lib().fp8_silu_mul_quant_dynamic(_ptr(gu), gu.stride(0), rows, cols, _ptr(y_out),
                                            y_out.stride(0) if y_out is not None else 0, _ptr(q), q.stride(0),
                                            _ptr(scale), _ptr(workspace), _stream()), "fp8_silu_mul_quant_dynamic")
    return q, scale, y_out
