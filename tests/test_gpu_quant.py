"""Quantization on the GPU vs the CPU oracle: bytes and scales bit-exact."""
import numpy as np
import pytest
import torch

import oracle
import fp8_w8a8_quantized_amd as fp8
from fp8_w8a8_quantized_amd import synth
from _helpers import say, dev_bf16, host_u8, host_f32, host_bf16_bits

pytestmark = pytest.mark.gpu


def _all_finite_bf16_upto_448():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = oracle.bf16_bits_to_f32(bits)
    keep = np.isfinite(x) & (np.abs(x) <= 448.0)
    return bits[keep]


def test_dynamic_exhaustive_bf16_scale_one():
    """Every finite bf16 with |v| <= 448 (448 itself included): amax = 448 so the
    scale is exactly 1 and every code is the plain e4m3fn encoding."""
    bits = _all_finite_bf16_upto_448()
    n = bits.size
    cols = 509                             # odd width: ragged row ends
    rows = -(-n // cols)
    pad = np.zeros(rows * cols, np.uint16); pad[:n] = bits
    x = pad.reshape(rows, cols)
    say("exhaustive bf16", x.shape)
    q, s = fp8.quant_dynamic(dev_bf16(x))
    torch.cuda.synchronize()
    assert host_f32(s)[0] == 1.0
    q_ref = oracle.quant_static(x, np.float32(1.0))
    assert np.array_equal(host_u8(q), q_ref)


@pytest.mark.parametrize("shape,outliers", [
    ((16, 4096), False), ((16, 4096), True), ((16, 14336), True),   # decode activations
    ((1, 4096), False), ((13, 4096), False), ((3, 1000), False),    # skinny / ragged
    ((300, 777), True), ((1024, 4096), True),                       # two-launch path
])
def test_dynamic_matches_oracle(shape, outliers):
    x = synth.activations(2, *shape, outliers=outliers)
    say("quant_dynamic", shape, outliers)
    q, s = fp8.quant_dynamic(dev_bf16(x))
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quant_dynamic(x)
    assert host_f32(s)[0] == s_ref
    assert np.array_equal(host_u8(q), q_ref)


def test_dynamic_strided_and_unaligned_layouts():
    x = synth.activations(4, 37, 300)
    big = torch.zeros((37, 333), dtype=torch.bfloat16, device="cuda")
    big[:, 5:305] = dev_bf16(x)
    xv = big[:, 5:305]                     # row pitch 333, base not 16-B aligned
    qbuf = torch.full((37, 321), 0xAA, dtype=torch.uint8, device="cuda")
    q = qbuf[:, 3:303]
    fp8.quant_dynamic(xv, q=q)
    torch.cuda.synchronize()
    q_ref, _ = oracle.quant_dynamic(x)
    host = host_u8(qbuf)
    assert np.array_equal(host[:, 3:303], q_ref)
    assert np.all(host[:, :3] == 0xAA) and np.all(host[:, 303:] == 0xAA)   # canaries intact


def test_dynamic_zero_tiny_and_empty():
    z = torch.zeros((16, 4096), dtype=torch.bfloat16, device="cuda")
    q, s = fp8.quant_dynamic(z)
    torch.cuda.synchronize()
    assert host_f32(s)[0] == 1.0 and np.all(host_u8(q) == 0)
    # tiny magnitudes: the scale is subnormal-adjacent; no flush to zero
    tiny = (synth.activations(5, 8, 256).astype(np.uint32) & 0x807F) | 0x0080   # exponent 1 (~1e-38)
    tiny = tiny.astype(np.uint16)
    q, s = fp8.quant_dynamic(dev_bf16(tiny))
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quant_dynamic(tiny)
    assert host_f32(s)[0] == s_ref and np.array_equal(host_u8(q), q_ref)
    e = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    q, s = fp8.quant_dynamic(e)
    torch.cuda.synchronize()
    assert host_f32(s)[0] == 1.0 and q.shape == (0, 64)


def test_static_saturates_and_matches_oracle():
    x = synth.activations(6, 64, 520, outliers=True)
    for sc in (0.01, 0.0371, 1.0, 3.5):
        s = torch.tensor([sc], dtype=torch.float32, device="cuda")
        q = fp8.quant_static(dev_bf16(x), s)
        torch.cuda.synchronize()
        q_ref = oracle.quant_static(x, np.float32(sc))
        assert np.array_equal(host_u8(q), q_ref), sc
        if sc <= 0.0371:   # |x| reaches ~90 with the outliers: these scales saturate
            assert np.sum((q_ref & 0x7F) == 0x7E) > 10


def test_static_exhaustive_bf16_unit_scale():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = oracle.bf16_bits_to_f32(bits)
    bits = bits[np.isfinite(x)].reshape(-1, 4)          # beyond 448 saturates
    s = torch.ones(1, dtype=torch.float32, device="cuda")
    q = fp8.quant_static(dev_bf16(bits), s)
    torch.cuda.synchronize()
    assert np.array_equal(host_u8(q), oracle.quant_static(bits, np.float32(1.0)))


@pytest.mark.parametrize("n,k,rowmul", [(1030, 4096, True), (6144, 4096, True), (64, 14336, False), (7, 33, True)])
def test_per_row_weight_quant_matches_oracle(n, k, rowmul):
    w = synth.weights(2, n, k, row_multipliers=rowmul)
    say("quant per row", n, k)
    q, s = fp8.quant_dynamic_per_row(dev_bf16(w))
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quant_weight(w, per_channel=True)
    assert np.array_equal(host_f32(s), s_ref)
    assert np.array_equal(host_u8(q), q_ref)


def test_per_tensor_weight_quant_matches_oracle():
    w = synth.weights(1, 4096, 4096)
    q, s = fp8.quant_weight(dev_bf16(w), per_channel=False)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quant_weight(w, per_channel=False)
    assert host_f32(s)[0] == s_ref[0]
    assert np.array_equal(host_u8(q), q_ref)


def test_prefill_activation_quant_full_size():
    """16384 x 4096 prefill activations (two-launch path), every byte."""
    x = synth.activations(3, 16384, 4096, outliers=True)
    say("prefill quant 16384x4096")
    q, s = fp8.quant_dynamic(dev_bf16(x))
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quant_dynamic(x)
    assert host_f32(s)[0] == s_ref
    assert np.array_equal(host_u8(q), q_ref)


def test_prefill_down_proj_quant_sampled_rows():
    """16384 x 14336: scale bit-exact over the whole tensor, bytes on sampled rows."""
    x = synth.activations(3, 16384, 14336, layer=0, sub=3, outliers=True)
    say("prefill quant 16384x14336")
    q, s = fp8.quant_dynamic(dev_bf16(x))
    torch.cuda.synchronize()
    s_ref = oracle.scale_from_amax(oracle.amax(oracle.bf16_bits_to_f32(x)))
    assert host_f32(s)[0] == s_ref
    rows = np.unique(np.concatenate([np.random.default_rng(0).integers(0, 16384, 256), np.arange(16128, 16384)]))
    qh = host_u8(q)
    assert np.array_equal(qh[rows], oracle.quant_static(x[rows], s_ref))


def test_quant_is_deterministic():
    x = dev_bf16(synth.activations(7, 2048, 4096, outliers=True))
    q1, s1 = fp8.quant_dynamic(x)
    q2, s2 = fp8.quant_dynamic(x)
    torch.cuda.synchronize()
    assert torch.equal(q1, q2) and torch.equal(s1, s2)


@pytest.mark.parametrize("shape", [(32, 4096), (32, 4104), (1, 131072), (1, 131080), (2, 65544), (16, 8192)])
@pytest.mark.parametrize("where", ["first", "last"])
def test_dynamic_one_and_two_launch_boundary(shape, where):
    """Either side of the one-launch limit (16384 units of 8 elements: 32 x 4096
    and 1 x 131072 take one launch, one unit more takes two), with the tensor's
    largest magnitude planted at its first or its last element, so the scale
    depends on the slot or block that holds it."""
    say("quant boundary", shape, where)
    x = synth.activations(9, *shape, outliers=False).copy()
    big = np.uint16(0xC2A0)  # bf16 -80.0, larger in magnitude than any generated value
    if where == "first":
        x[0, 0] = big
    else:
        x[-1, -1] = big
    q, s = fp8.quant_dynamic(dev_bf16(x))
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quant_dynamic(x)
    assert s_ref == np.float32(80.0) / np.float32(448.0)
    assert host_f32(s)[0] == s_ref
    assert np.array_equal(host_u8(q), q_ref)


@pytest.mark.parametrize("n,k", [(28672, 4096), (4096, 14336)])
def test_per_channel_weight_quant_full_llama_shapes(n, k):
    """Per-output-channel weight quantization at the two largest Llama-3-8B
    shapes the benchmark times, codes and scales bit for bit."""
    say("weight quant per channel", n, k)
    w = synth.weights(2, n, k, row_multipliers=True)
    q, s = fp8.quant_weight(dev_bf16(w), True)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quant_weight(w, True)
    assert np.array_equal(host_f32(s), s_ref)
    assert np.array_equal(host_u8(q), q_ref)


def test_static_quant_prefill_size():
    """Static quantization at the prefill size the benchmark times (16384 x
    4096, the benchmark's scale 0.05): every code bit for bit, saturation
    included."""
    say("static quant 16384 x 4096")
    x = synth.activations(3, 16384, 4096, outliers=True)
    s = torch.tensor([0.05], dtype=torch.float32, device="cuda")
    q = fp8.quant_static(dev_bf16(x), s)
    torch.cuda.synchronize()
    assert np.array_equal(host_u8(q), oracle.quant_static(x, np.float32(0.05)))


@pytest.mark.timeout(600)
def test_quantizers_past_4_gib_sampled_rows():
    """A bf16 tensor of 65536 x 32776 (4.3 GB, past 4 GiB): beyond the
    buffer-load batches' 2 GiB range, so the dynamic (two launches),
    static and per-row quantizers read it with 64-bit row addresses.  The
    tensor is drawn on the device (N(0,1), far below 80 at this size) with
    -80 planted in its last element, so the dynamic scale is fl32(80/448).
    Rows on both sides of the 2 GiB and 4 GiB byte marks, and the first and
    last rows, are compared with the oracle byte for byte; the per-row
    scales of those rows too."""
    rows, cols = 65536, 32776
    gen = torch.Generator(device="cuda")
    gen.manual_seed(12)
    x = torch.randn((rows, cols), generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    x[-1, -1] = -80.0
    torch.cuda.synchronize()
    row_bytes = cols * 2
    marks = [(1 << 31) // row_bytes, (1 << 32) // row_bytes]
    sample = sorted({0, 1, rows - 2, rows - 1, *[r + d for r in marks for d in (-1, 0, 1)]})
    say("4 GiB tensor, sampled rows", sample)
    xs = host_bf16_bits(x[sample])
    s_ref = oracle.scale_from_amax(np.float32(80.0))

    q, s = fp8.quant_dynamic(x)
    torch.cuda.synchronize()
    assert host_f32(s)[0] == s_ref
    assert np.array_equal(host_u8(q[sample]), oracle.quant_static(xs, s_ref))
    del q

    s_static = torch.tensor([0.05], dtype=torch.float32, device="cuda")
    q = fp8.quant_static(x, s_static)
    torch.cuda.synchronize()
    assert np.array_equal(host_u8(q[sample]), oracle.quant_static(xs, np.float32(0.05)))
    del q

    q, s_rows = fp8.quant_weight(x, True)
    torch.cuda.synchronize()
    q_ref, s_rows_ref = oracle.quant_weight(xs, True)
    assert np.array_equal(host_f32(s_rows)[sample], s_rows_ref)
    assert np.array_equal(host_u8(q[sample]), q_ref)


@pytest.mark.timeout(300)
def test_per_row_quantizer_past_2_pow_24_rows():
    """16,777,221 rows of 16 (512 MiB of bf16): one 256-thread workgroup per
    row would pass 2^32 threads in one launch, so past 2^20 rows each
    workgroup takes several rows.  Rows on both sides of the 2^20 and 2^24
    marks (the first rows handled by a workgroup's second and 17th turn),
    the first and the last rows are compared with the oracle: codes and
    scales bit for bit."""
    rows, cols = (1 << 24) + 5, 16
    gen = torch.Generator(device="cuda")
    gen.manual_seed(23)
    x = torch.randn((rows, cols), generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    torch.cuda.synchronize()
    sample = sorted({0, 1, rows - 2, rows - 1, *[r + d for r in (1 << 20, 1 << 24) for d in (-1, 0, 1)]})
    say("per-row quantizer, rows", rows, "sampled", sample)
    xs = host_bf16_bits(x[sample])
    q, s_rows = fp8.quant_weight(x, True)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quant_weight(xs, True)
    assert np.array_equal(host_f32(s_rows[sample]), s_ref)
    assert np.array_equal(host_u8(q[sample]), q_ref)
