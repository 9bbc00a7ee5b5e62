"""e5m2 (the extension the compressed-tensors fp8 page names) on the GPU vs
the CPU oracle: codes and scales bit-exact, GEMMs with any mix of e4m3 and
e5m2 operands within the same tolerance as e4m3."""
import numpy as np
import pytest
import torch

import oracle
import fp8_w8a8_quantized_amd as fp8
from fp8_w8a8_quantized_amd import synth
from _helpers import say, dev_bf16, host_u8, host_f32, host_bf16_bits, assert_gemm_close

pytestmark = pytest.mark.gpu


def test_e5m2_dynamic_exhaustive_bf16_scale_one():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = oracle.bf16_bits_to_f32(bits)
    keep = bits[np.isfinite(x) & (np.abs(x) <= 57344.0)]
    keep = np.concatenate([keep, oracle.f32_to_bf16_bits(np.array([57344.0], np.float32))])
    cols = 509
    rows = -(-keep.size // cols)
    pad = np.zeros(rows * cols, np.uint16); pad[:keep.size] = keep
    xb = pad.reshape(rows, cols)
    say("e5m2 exhaustive", xb.shape)
    q, s = fp8.quant_dynamic(dev_bf16(xb), fmt="e5m2")
    torch.cuda.synchronize()
    assert host_f32(s)[0] == 1.0
    assert np.array_equal(host_u8(q), oracle.quant_static(xb, np.float32(1.0), "e5m2"))


@pytest.mark.parametrize("shape", [(16, 4096), (16, 14336), (300, 4096), (5, 1003)])
def test_e5m2_dynamic_matches_oracle(shape):
    x = synth.activations(61, *shape, outliers=True)
    say("e5m2 dynamic", shape)
    q, s = fp8.quant_dynamic(dev_bf16(x), fmt="e5m2")
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quant_dynamic(x, "e5m2")
    assert host_f32(s)[0] == np.float32(s_ref)
    assert np.array_equal(host_u8(q), q_ref)


def test_e5m2_static_saturates():
    x = synth.activations(62, 64, 1000, outliers=True)
    s = torch.tensor([2.0 ** -12], dtype=torch.float32, device="cuda")    # |x| up to ~100 -> far past 57344
    q = fp8.quant_static(dev_bf16(x), s, fmt="e5m2")
    torch.cuda.synchronize()
    ref = oracle.quant_static(x, np.float32(2.0 ** -12), "e5m2")
    assert np.array_equal(host_u8(q), ref)
    assert np.any((ref & 0x7F) == 0x7B)


@pytest.mark.parametrize("per_channel", [True, False])
def test_e5m2_weight_quant(per_channel):
    w = synth.weights(63, 1030, 4096, row_multipliers=True)
    q, s = fp8.quant_weight(dev_bf16(w), per_channel, fmt="e5m2")
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quant_weight(w, per_channel, "e5m2")
    assert np.array_equal(host_f32(s).reshape(-1), s_ref.reshape(-1))
    assert np.array_equal(host_u8(q), q_ref)


FMTS = [("e5m2", "e5m2"), ("e4m3", "e5m2"), ("e5m2", "e4m3")]


def _gemm_case(m, k, n, fa, fw, per_channel, accum, seed):
    x = synth.activations(seed, m, k, outliers=True)
    w = synth.weights(seed, n, k, row_multipliers=per_channel)
    aq, sa = oracle.quant_dynamic(x, fa)
    wq, sw = oracle.quant_weight(w, per_channel, fw)
    out = fp8.scaled_mm(torch.from_numpy(aq).cuda(), torch.from_numpy(wq).cuda(),
                        torch.tensor([sa], dtype=torch.float32, device="cuda"), torch.from_numpy(sw).cuda(),
                        per_channel, accum=accum, fmt_a=fa, fmt_w=fw)
    torch.cuda.synchronize()
    ref = oracle.scaled_mm(aq, wq, sa, sw, per_channel, fmt_a=fa, fmt_w=fw)
    assert_gemm_close(host_bf16_bits(out), ref, aq, sa, wq, sw, per_channel, accum=accum, fmt_a=fa, fmt_w=fw)


@pytest.mark.parametrize("fa,fw", FMTS)
@pytest.mark.parametrize("m,k,n", [(16, 4096, 1030), (3, 4096, 4100), (7, 1000, 33), (40, 4096, 300),
                                   # K >= 8192 (interleaved K steps) and/or >= 32 MiB of weights
                                   # (non-temporal loads): every variant of the skinny kernel
                                   (3, 8208, 257), (4, 8192, 4100), (5, 4096, 8200), (6, 2048, 16400),
                                   # 16 < M <= 64 on wide weights: the wide kernel (on a 256-CU part)
                                   (20, 1024, 28680), (36, 1024, 14400)])
def test_e5m2_skinny_gemm(fa, fw, m, k, n):
    say("e5m2 skinny", fa, fw, m, k, n)
    _gemm_case(m, k, n, fa, fw, True, "fp32", 64)


@pytest.mark.parametrize("fa,fw", FMTS)
@pytest.mark.parametrize("accum", ["fp32", "fp8"])
def test_e5m2_mfma_gemm(fa, fw, accum):
    say("e5m2 mfma", fa, fw, accum)
    _gemm_case(320, 4096, 1040, fa, fw, True, accum, 65)
