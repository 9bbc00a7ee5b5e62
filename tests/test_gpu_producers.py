"""Producer-fused quantization on the GPU vs the CPU oracle, from the same
seeded inputs: the residual add, the normalized / activated bf16 values
(float64 on both sides, one rounding to bf16), the codes and the scale are
all compared bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import fp8_w8a8_quantized_amd as fp8
from fp8_w8a8_quantized_amd import synth
from _helpers import say, dev_bf16, host_u8, host_f32, host_bf16_bits

pytestmark = pytest.mark.gpu


def _pitched(bits, pitch):
    """A device bf16 view [rows, cols] inside a wider [rows, pitch] buffer."""
    rows, cols = bits.shape
    buf = np.zeros((rows, pitch), np.uint16)
    buf[:, :cols] = bits
    return dev_bf16(buf)[:, :cols]


def _check_quant(y_ref_bits, q, s):
    q_ref, s_ref = oracle.quant_dynamic(y_ref_bits)
    assert host_f32(s)[0] == np.float32(s_ref)
    assert np.array_equal(host_u8(q), q_ref)


@pytest.mark.parametrize("rows,cols,pitch,with_delta", [
    (16, 4096, 4096, True),      # decode, one-launch quantization
    (16, 4096, 4096, False),
    (300, 4096, 4096, True),     # two-launch quantization
    (2500, 512, 520, True),      # more rows than row groups: 2 or 3 rows per workgroup
    (2500, 512, 512, False),
    (5, 1003, 1011, True),       # ragged row ends, odd pitch
    (1, 14336, 14336, True),
])
def test_add_rmsnorm_quant(rows, cols, pitch, with_delta):
    say("add_rmsnorm_quant", rows, cols, pitch, with_delta)
    h = synth.activations(41, rows, cols, outliers=True)
    d = synth.activations(42, rows, cols, outliers=False)
    hd = _pitched(h, pitch)
    dd = _pitched(d, pitch) if with_delta else None
    h_out = _pitched(np.zeros_like(h), pitch) if with_delta else None
    y = torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda")
    q, s, h2, _ = fp8.add_rmsnorm_quant(hd, dd, h_out=h_out, y_out=y)
    torch.cuda.synchronize()
    if with_delta:
        h_ref = oracle.add_bf16(h, d)
        assert np.array_equal(host_bf16_bits(h2), h_ref)
    else:
        h_ref = h
    y_ref = oracle.rmsnorm(h_ref, 1e-5)
    dist = oracle.bf16_ulp_distance(host_bf16_bits(y), y_ref)
    assert dist.max() == 0, (int(dist.max()), int(np.count_nonzero(dist)))
    _check_quant(y_ref, q, s)
    # the optional copy does not change the codes
    q2, s2, _, _ = fp8.add_rmsnorm_quant(hd, dd, h_out=torch.empty_like(hd) if with_delta else None)
    torch.cuda.synchronize()
    assert torch.equal(q2, q) and torch.equal(s2, s)


@pytest.mark.parametrize("rows,cols,pitch", [
    (16, 14336, 2 * 14336),      # decode gate_up output
    (64, 14336, 2 * 14336),
    (3, 1001, 2 * 1001 + 5),     # ragged, odd pitch (unaligned up half)
    (300, 14336, 2 * 14336),     # >= 4 Mi elements: the float32 path with its float64 fallback
    (4100, 1030, 2 * 1030 + 3),  # the same, unaligned
])
def test_silu_mul_quant(rows, cols, pitch):
    say("silu_mul_quant", rows, cols, pitch)
    gu = synth.activations(43, rows, 2 * cols, outliers=True)
    gud = _pitched(gu, pitch)
    y = torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda")
    q, s, _ = fp8.silu_mul_quant(gud, y_out=y)
    torch.cuda.synchronize()
    y_ref = oracle.silu_mul(gu, cols)
    dist = oracle.bf16_ulp_distance(host_bf16_bits(y), y_ref)
    assert dist.max() == 0, (int(dist.max()), int(np.count_nonzero(dist)))
    _check_quant(y_ref, q, s)
    q2, s2, _ = fp8.silu_mul_quant(gud)
    torch.cuda.synchronize()
    assert torch.equal(q2, q) and torch.equal(s2, s)


def test_producers_empty():
    h = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    q, s, _, _ = fp8.add_rmsnorm_quant(h)
    gu = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    q2, s2, _ = fp8.silu_mul_quant(gu)
    torch.cuda.synchronize()
    assert host_f32(s)[0] == 1.0 and host_f32(s2)[0] == 1.0


def _chunked_ref(fn, rows, chunk=1024):
    """The oracle's bf16 output of fn(row range) over all rows, in chunks of
    rows (bounded host memory), as one array."""
    return np.concatenate([fn(r0, min(r0 + chunk, rows)) for r0 in range(0, rows, chunk)])


@pytest.mark.parametrize("which", ["add_rmsnorm", "silu_mul"])
def test_producers_at_prefill_size(which):
    """The fused producers at the prefill sizes the benchmark times (16384 x
    4096 normalization with a residual add; 16384 x 14336 SiLU*mul): the
    scale over the whole tensor, h' and the codes on sampled rows plus the
    last 64, bit for bit."""
    m = 16384
    rows = np.unique(np.concatenate([np.random.default_rng(7).integers(0, m, 96), np.arange(m - 64, m)]))
    if which == "add_rmsnorm":
        k = 4096
        say("add_rmsnorm_quant at", m, "x", k)
        h = synth.activations(44, m, k, outliers=True)
        d = synth.activations(45, m, k, outliers=False)
        hd, dd = dev_bf16(h), dev_bf16(d)
        q, s, h2, _ = fp8.add_rmsnorm_quant(hd, dd, h_out=torch.empty_like(hd))
        torch.cuda.synchronize()
        h_ref = oracle.add_bf16(h, d)
        assert np.array_equal(host_bf16_bits(h2)[rows], h_ref[rows])
        y_ref = _chunked_ref(lambda a, b: oracle.rmsnorm(h_ref[a:b], 1e-5), m)
    else:
        k = 14336
        say("silu_mul_quant at", m, "x", k)
        gu = synth.activations(46, m, 2 * k, outliers=True)
        q, s, _ = fp8.silu_mul_quant(dev_bf16(gu))
        torch.cuda.synchronize()
        y_ref = _chunked_ref(lambda a, b: oracle.silu_mul(gu[a:b], k), m)
    s_ref = oracle.scale_from_amax(oracle.amax(oracle.bf16_bits_to_f32(y_ref)))
    assert host_f32(s)[0] == s_ref
    assert np.array_equal(host_u8(q)[rows], oracle.quant_static(y_ref[rows], s_ref))


def _device_normal(shape, seed):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    return torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)


def _sample_rows(rows, row_bytes):
    marks = [(1 << 31) // row_bytes, (1 << 32) // row_bytes]
    return sorted({0, 1, rows - 2, rows - 1, *[r + d for r in marks for d in (-1, 0, 1) if 0 <= r + d < rows]})


@pytest.mark.timeout(600)
def test_producers_past_4_gib_sampled_rows():
    """Both fused producers on inputs past 4 GiB, read with 64-bit row
    addresses.  The inputs are drawn on the device (N(0,1)) with a planted
    row that holds the tensor's largest value: for add + RMS norm, a last row
    whose only nonzero entry normalizes to about sqrt(cols) = 181 (other rows
    stay near 5); for SiLU*mul, gate = up = 80 in the last row (6400; other
    products stay below about 40).  The oracle computes that row's values, so
    it knows the scale, and compares the sampled rows' outputs and codes
    byte for byte."""
    rows, cols = 65536, 32776
    h = _device_normal((rows, cols), 21)
    d = _device_normal((rows, cols), 22)
    h[-1].zero_(); d[-1].zero_()
    h[-1, 5] = 100.0
    torch.cuda.synchronize()
    sample = _sample_rows(rows, cols * 2)
    say("add_rmsnorm_quant past 4 GiB, sampled rows", sample)
    idx = torch.tensor(sample, device="cuda")
    h_rows, d_rows = host_bf16_bits(h[idx]), host_bf16_bits(d[idx])
    h_out = torch.empty_like(h)
    q, s, _, _ = fp8.add_rmsnorm_quant(h, d, h_out=h_out)
    torch.cuda.synchronize()
    del h, d
    hs_ref = oracle.add_bf16(h_rows, d_rows)
    y_ref = oracle.rmsnorm(hs_ref, 1e-5)
    s_ref = oracle.scale_from_amax(np.max(np.abs(oracle.bf16_bits_to_f32(y_ref[-1]))))
    assert host_f32(s)[0] == s_ref
    assert np.array_equal(host_bf16_bits(h_out[idx]), hs_ref)
    assert np.array_equal(host_u8(q[idx]), oracle.quant_static(y_ref, s_ref))
    del h_out, q

    rows, cols = 40000, 28680
    gu = _device_normal((rows, 2 * cols), 23)
    gu[-1, 3] = 80.0
    gu[-1, cols + 3] = 80.0
    torch.cuda.synchronize()
    sample = _sample_rows(rows, 2 * cols * 2)
    say("silu_mul_quant past 4 GiB, sampled rows", sample)
    idx = torch.tensor(sample, device="cuda")
    gu_rows = host_bf16_bits(gu[idx])
    q, s, _ = fp8.silu_mul_quant(gu)
    torch.cuda.synchronize()
    del gu
    y_ref = oracle.silu_mul(gu_rows, cols)
    s_ref = oracle.scale_from_amax(np.max(np.abs(oracle.bf16_bits_to_f32(y_ref[-1]))))
    assert host_f32(s)[0] == s_ref
    assert np.array_equal(host_u8(q[idx]), oracle.quant_static(y_ref, s_ref))
