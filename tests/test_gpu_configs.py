"""The five workloads at their real sizes, GPU vs the CPU oracle.

Llama-3-8B decoder linears as (K, N): QKV 4096->6144, O 4096->4096, gate_up
4096->28672, down 14336->4096; Mistral-7B-shaped skinny GEMMs at unaligned N.
Quantized bytes and scales are compared bit for bit; GEMM outputs within
the element-wise tolerance.  Prefill outputs (16384 rows) are checked on a
sample of rows plus the whole last 256-row tile.
"""
import numpy as np
import pytest
import torch

import oracle
import fp8_w8a8_quantized_amd as fp8
from fp8_w8a8_quantized_amd import synth
from _helpers import say, dev_bf16, host_u8, host_f32, host_bf16_bits, assert_gemm_close

pytestmark = pytest.mark.gpu


def _linear_case(cfg, m, k, n, per_channel, outliers, rowmul, sub, rows=None, accum="fp32", fmt="e4m3"):
    x = synth.activations(cfg, m, k, sub=sub, outliers=outliers)
    w = synth.weights(cfg, n, k, sub=sub, row_multipliers=rowmul)
    xd, wd = dev_bf16(x), dev_bf16(w)
    w_q, s_w = fp8.quant_weight(wd, per_channel, fmt=fmt)
    a_q, s_a = fp8.quant_dynamic(xd, fmt=fmt)
    out = fp8.scaled_mm(a_q, w_q, s_a, s_w, per_channel, accum=accum, fmt_a=fmt, fmt_w=fmt)
    torch.cuda.synchronize()
    wq, sw = oracle.quant_weight(w, per_channel, fmt)
    assert np.array_equal(host_f32(s_w), sw) and np.array_equal(host_u8(w_q), wq)
    sa = oracle.scale_from_amax(oracle.amax(oracle.bf16_bits_to_f32(x)), fmt)
    assert host_f32(s_a)[0] == sa
    xs = x if rows is None else x[rows]
    aq = oracle.quant_static(xs, sa, fmt)
    assert np.array_equal(host_u8(a_q) if rows is None else host_u8(a_q)[rows], aq)
    ref = oracle.scaled_mm(aq, wq, sa, sw, per_channel, fmt_a=fmt, fmt_w=fmt)
    ob = host_bf16_bits(out)
    stat = assert_gemm_close(ob if rows is None else ob[rows], ref, aq, sa, wq, sw, per_channel, accum=accum,
                             fmt_a=fmt, fmt_w=fmt)
    if accum == "fp32":
        say(f"  ok (max rel err {stat:.3g})")
    else:
        n_big = int(np.count_nonzero(np.abs(ref) > 1e-3))
        say(f"  ok (within the fp8-accumulation bound; relative clause broken on {stat} of {n_big} "
            f"elements with |ref| > 1e-3)")


def test_single_linear_per_tensor_16x4096x4096():
    say("16 x 4096 -> 4096 per-tensor")
    _linear_case(1, 16, 4096, 4096, False, False, False, 0)


@pytest.mark.parametrize("sub,name,k,n", [(i,) + s for i, s in enumerate(synth.LLAMA3_8B_LINEARS)])
def test_llama3_8b_decode_channelwise(sub, name, k, n):
    say(f"decode {name} 16 x {k} -> {n} channelwise")
    _linear_case(2, 16, k, n, True, True, True, sub)


@pytest.mark.parametrize("accum", ["fp32", "fp8"])
@pytest.mark.parametrize("sub,name,k,n", [(i,) + s for i, s in enumerate(synth.LLAMA3_8B_LINEARS)])
def test_llama3_8b_prefill_channelwise_sampled(sub, name, k, n, accum):
    m = 16384
    rows = np.unique(np.concatenate([np.random.default_rng(sub).integers(0, m, 256), np.arange(m - 256, m)]))
    say(f"prefill {name} {m} x {k} -> {n} channelwise, {rows.size} rows checked, accum {accum}")
    _linear_case(3, m, k, n, True, True, True, sub, rows=rows, accum=accum)


@pytest.mark.parametrize("sub,name,k,n", [(i,) + s for i, s in enumerate(synth.LLAMA3_8B_LINEARS)])
def test_llama3_8b_e5m2_decode_and_prefill_sampled(sub, name, k, n):
    """e5m2 activations and weights (channelwise, exact sums) at the layer's
    decode size in full and at its prefill size on sampled rows: the problems
    the benchmark times for the e5m2 path."""
    say(f"e5m2 decode {name} 16 x {k} -> {n}")
    _linear_case(2, 16, k, n, True, True, True, sub, fmt="e5m2")
    m = 16384
    rows = np.unique(np.concatenate([np.random.default_rng(100 + sub).integers(0, m, 128), np.arange(m - 64, m)]))
    say(f"e5m2 prefill {name} {m} x {k} -> {n}, {rows.size} rows checked")
    _linear_case(3, m, k, n, True, True, True, sub, rows=rows, fmt="e5m2")


@pytest.mark.parametrize("m", synth.MISTRAL_7B_SKINNY_M)
def test_mistral_7b_unaligned_per_tensor(m):
    for j, (k, n) in enumerate(synth.MISTRAL_7B_KN):
        say(f"mistral M={m} {k} -> {n} per-tensor")
        _linear_case(4, m, k, n, False, False, False, 10 * m + j)
