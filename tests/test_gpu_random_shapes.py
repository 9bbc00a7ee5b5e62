"""Scaled GEMM on seeded random problems vs the exact CPU oracle.

Each case draws M, N, K, the row pitches of both operands and of the output,
the scale mode, a bias, the operand formats and the accumulation mode from a
fixed seed. Together the cases cross every dispatch path of the library:
- the one-block skinny kernel (M <= 16);
- the multi-block skinny kernel (16 < M <= 64, in one or two grid rows);
- the byte-granular kernel (K % 16 != 0 or unaligned pitches);
- the matrix-core kernel (M > 64 with enough output tiles), with vector and
  2-byte output stores, and the multi-block skinny kernel for the 64 < M <= 256
  problems too small for its tiles;
- on wide weights (N of 14305 and more, the last six cases, on a 256-CU
  part): the two-block skinny kernel (M <= 16) and the wide skinny kernel
  (16 < M <= 64), or the multi-block or byte-granular one where those do not
  apply.
The operands are quantized from the seeded generators on each side
independently, and the GPU's codes must equal the oracle's byte for byte.
"""
import numpy as np
import pytest
import torch

import oracle
import fp8_w8a8_quantized_amd as fp8
from fp8_w8a8_quantized_amd import synth
from _helpers import say, dev_bf16, host_u8, host_f32, host_bf16_bits, assert_gemm_close

pytestmark = pytest.mark.gpu

CONFIG = 7  # seed stream of these cases


def _cases(n_cases=30, seed=20261202):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n_cases):
        band = i % 3
        m = int(rng.integers(1, 17) if band == 0 else rng.integers(17, 65) if band == 1 else rng.integers(65, 321))
        aligned = rng.random() < 0.6
        k = int(rng.integers(1, 125) * 16 if aligned else rng.integers(1, 2000))
        n = int(rng.integers(1, 2600))
        pad_a = int(rng.choice([0, 0, 16, 48, 5]))
        pad_w = int(rng.choice([0, 0, 32, 7]))
        pad_o = int(rng.choice([0, 0, 8, 3]))
        per_channel = bool(rng.random() < 0.6)
        with_bias = bool(rng.random() < 0.5)
        fmt_a, fmt_w = [("e4m3", "e4m3"), ("e4m3", "e4m3"), ("e4m3", "e4m3"), ("e5m2", "e4m3"),
                        ("e4m3", "e5m2"), ("e5m2", "e5m2")][int(rng.integers(0, 6))]
        accum = "fp8" if (m > 64 and rng.random() < 0.4) else "fp32"
        out.append((i, m, n, k, pad_a, pad_w, pad_o, per_channel, with_bias, fmt_a, fmt_w, accum))
    return out


def _wide_cases(n_cases=6, seed=20261203):
    """Wide weights with short K (so the oracle stays quick): M <= 16, 17-32
    on N >= 28672, and 33-64 on N >= 14336."""
    rng = np.random.default_rng(seed)
    out = []
    for j in range(n_cases):
        band = j % 3
        m = int(rng.integers(1, 17) if band == 0 else rng.integers(17, 33) if band == 1 else rng.integers(33, 65))
        lo = 28672 if band == 1 else 14305
        n = int(rng.integers(lo, 32001))
        aligned = rng.random() < 0.8
        k = int(rng.integers(1, 33) * 16 if aligned else rng.integers(1, 520))
        pad_a = int(rng.choice([0, 16, 48]))
        pad_w = int(rng.choice([0, 32, 7]))
        pad_o = int(rng.choice([0, 8, 3]))
        per_channel = bool(rng.random() < 0.6)
        with_bias = bool(rng.random() < 0.5)
        fmt_a, fmt_w = [("e4m3", "e4m3"), ("e4m3", "e4m3"), ("e5m2", "e4m3"), ("e4m3", "e5m2")][int(rng.integers(0, 4))]
        out.append((30 + j, m, n, k, pad_a, pad_w, pad_o, per_channel, with_bias, fmt_a, fmt_w, "fp32"))
    return out


def _pitched_codes(codes, pad):
    """A device uint8 view [rows, cols] inside a [rows, cols + pad] buffer."""
    rows, cols = codes.shape
    buf = torch.zeros((rows, cols + pad), dtype=torch.uint8, device="cuda")
    view = buf[:, :cols]
    view.copy_(torch.from_numpy(np.ascontiguousarray(codes)).cuda())
    return view


@pytest.mark.parametrize("case", _cases() + _wide_cases(), ids=lambda c: f"c{c[0]}-m{c[1]}-n{c[2]}-k{c[3]}")
def test_random_problem(case):
    i, m, n, k, pad_a, pad_w, pad_o, per_channel, with_bias, fmt_a, fmt_w, accum = case
    say("random gemm", case)
    x = synth.activations(CONFIG, m, k, sub=i, outliers=(i % 2 == 0))
    w = synth.weights(CONFIG, n, k, sub=i, row_multipliers=per_channel)
    b = synth.bias(CONFIG, n, sub=i) if with_bias else None
    # quantization on both sides, compared byte for byte
    a_q_d, s_a = fp8.quant_dynamic(dev_bf16(x), fmt=fmt_a)
    w_q_d, s_w = fp8.quant_weight(dev_bf16(w), per_channel, fmt=fmt_w)
    aq, sa = oracle.quant_dynamic(x, fmt_a)
    wq, sw = oracle.quant_weight(w, per_channel, fmt_w)
    torch.cuda.synchronize()
    assert host_f32(s_a)[0] == sa and np.array_equal(host_u8(a_q_d), aq)
    assert np.array_equal(host_f32(s_w), sw) and np.array_equal(host_u8(w_q_d), wq)
    # the same codes at the drawn pitches, and an output view with canaries past N
    a_q = _pitched_codes(aq, pad_a)
    w_q = _pitched_codes(wq, pad_w)
    obuf = torch.full((m, n + pad_o), -5.0, dtype=torch.bfloat16, device="cuda")
    out = obuf[:, :n]
    bias = dev_bf16(b) if b is not None else None
    fp8.scaled_mm(a_q, w_q, s_a, s_w, per_channel, bias, out=out, accum=accum, fmt_a=fmt_a, fmt_w=fmt_w)
    torch.cuda.synchronize()
    ref = oracle.scaled_mm(aq, wq, sa, sw, per_channel, b, fmt_a=fmt_a, fmt_w=fmt_w)
    assert_gemm_close(host_bf16_bits(out), ref, aq, sa, wq, sw, per_channel, bias_bits=b, accum=accum,
                      fmt_a=fmt_a, fmt_w=fmt_w)
    if pad_o:  # the columns past N keep their canary (bf16 -5.0)
        assert np.all(host_bf16_bits(obuf)[:, n:] == 0xC0A0)
