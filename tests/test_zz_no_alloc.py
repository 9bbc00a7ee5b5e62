"""The no-allocation linear (fp8_linear_dynamic_noalloc) against the
workspace one (fp8_linear_dynamic), through the C ABI: outputs must be
identical bit for bit (the same kernels), on two calls in a row with the
second smaller, so the second call finds the first one's data in the
library's scratch array.  Both paths are also checked against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import fp8_w8a8_quantized_amd as fp8
from fp8_w8a8_quantized_amd import synth
from _helpers import say, dev_bf16, host_u8, host_f32, host_bf16_bits, assert_gemm_close

pytestmark = pytest.mark.gpu


def _case(seed, m, k, n, per_channel):
    x = synth.activations(seed, m, k, outliers=True)
    w = synth.weights(seed, n, k, row_multipliers=per_channel)
    b = synth.bias(seed, n)
    w_q, s_w = fp8.quant_weight(dev_bf16(w), per_channel)
    xd, bd = dev_bf16(x), dev_bf16(b)
    # reference: the entry point with a caller workspace
    out_ws, aq_ws, sa_ws = fp8.linear_dynamic(xd, w_q, s_w, per_channel, bd, workspace=fp8.new_linear_workspace())
    # no allocation: every output preallocated, no workspace
    a_q = torch.empty((m, k), dtype=torch.uint8, device="cuda")
    s_a = torch.empty(1, dtype=torch.float32, device="cuda")
    out = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    fp8.linear_dynamic_noalloc(xd, w_q, s_w, per_channel, bd, a_q, s_a, out)
    torch.cuda.synchronize()
    assert torch.equal(out, out_ws) and torch.equal(a_q, aq_ws) and torch.equal(s_a, sa_ws)
    aq, sa = oracle.quant_dynamic(x)
    wq, sw = oracle.quant_weight(w, per_channel)
    assert host_f32(s_a)[0] == sa and np.array_equal(host_u8(a_q), aq)
    ref = oracle.scaled_mm(aq, wq, sa, sw, per_channel, b)
    assert_gemm_close(host_bf16_bits(out), ref, aq, sa, wq, sw, per_channel, bias_bits=b)


@pytest.mark.parametrize("first,second", [
    # two-launch quantization (per-block maxima in the scratch) then a smaller one
    ((300, 4096, 640, True), (130, 1024, 200, False)),
    # the decode sizes: the down projection's input (two launches) then the one-launch size
    ((16, 14336, 1024, True), (3, 4096, 1030, False)),
])
def test_noalloc_matches_workspace_entry_point_twice(first, second):
    for i, (m, k, n, pc) in enumerate((first, second)):
        say(f"noalloc call {i}: {m} x {k} -> {n} {'channelwise' if pc else 'per tensor'}")
        _case(40 + i, m, k, n, pc)


@pytest.mark.parametrize("m,k,n", [(16, 4096, 1030), (16, 14336, 512), (300, 1024, 520)])
def test_noalloc_captured_in_a_graph(m, k, n):
    """The callers this entry point is for capture it into HIP graphs: one
    capture, four replays with eager work between them (output clears, a new
    input), each replay bit-identical to the workspace entry point called
    eagerly on the same input."""
    say("noalloc graph", m, k, n)
    w_q, s_w = fp8.quant_weight(dev_bf16(synth.weights(44, n, k, row_multipliers=True)), True)
    bd = dev_bf16(synth.bias(44, n))
    x = dev_bf16(synth.activations(44, m, k, outliers=True))
    x2 = dev_bf16(synth.activations(45, m, k, outliers=False, scale=3.0))
    a_q = torch.empty((m, k), dtype=torch.uint8, device="cuda")
    s_a = torch.empty(1, dtype=torch.float32, device="cuda")
    out = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    for _ in range(2):  # warm up outside the capture
        fp8.linear_dynamic_noalloc(x, w_q, s_w, True, bd, a_q, s_a, out)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fp8.linear_dynamic_noalloc(x, w_q, s_w, True, bd, a_q, s_a, out)
    torch.cuda.synchronize()
    ws = fp8.new_linear_workspace()
    refs = []
    for xi in (x, x2):
        o, q, s = fp8.linear_dynamic(xi, w_q, s_w, True, bd, workspace=ws)
        torch.cuda.synchronize()
        refs.append((o.clone(), q.clone(), s.clone()))
    x_orig = x.clone()
    for rep in range(4):
        a_q.zero_(); s_a.zero_(); out.zero_()
        x.copy_(x2 if rep >= 2 else x_orig)  # the graph reads whatever the buffer holds
        g.replay()
        torch.cuda.synchronize()
        want = refs[1] if rep >= 2 else refs[0]
        assert torch.equal(out.view(torch.int16), want[0].view(torch.int16)), rep
        assert torch.equal(a_q, want[1]), rep
        assert torch.equal(s_a, want[2]), rep
