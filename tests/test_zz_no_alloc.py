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
