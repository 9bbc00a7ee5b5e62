"""The layer captured into a HIP graph replays bit-identically to eager calls.

The C ABI never allocates, synchronizes or reads device memory on the host,
so a quantize + scaled GEMM pair can be captured once and replayed.  Each
replay is checked against eager results, with eager work (buffer clears,
new input values) between replays.
"""
import numpy as np
import pytest
import torch

import fp8_w8a8_quantized_amd as fp8
from fp8_w8a8_quantized_amd import synth
from _helpers import say, dev_bf16

pytestmark = pytest.mark.gpu


def _eager(x, w_q, s_w, ws, accum):
    a_q, s_a = fp8.quant_dynamic(x, workspace=ws)
    out = fp8.scaled_mm(a_q, w_q, s_a, s_w, True, accum=accum)
    torch.cuda.synchronize()
    return a_q.clone(), s_a.clone(), out.clone()


@pytest.mark.parametrize("m,k,n,accum", [(16, 4096, 1030, "fp32"), (16, 14336, 512, "fp32"),
                                         (300, 1024, 520, "fp32"), (300, 1024, 520, "fp8"),
                                         (2048, 4096, 1024, "fp32"),
                                         # a mid-M problem on the skinny kernel (two grid rows of M),
                                         # and 128 x 128 tiles with two workgroups on some CUs
                                         (128, 4096, 4096, "fp8"), (1024, 1024, 6144, "fp32")])
def test_graph_replay_matches_eager(m, k, n, accum):
    say("graph", m, k, n, accum)
    w_q, s_w = fp8.quant_weight(dev_bf16(synth.weights(7, n, k, row_multipliers=True)), True)
    x = dev_bf16(synth.activations(7, m, k, outliers=True))
    ws = fp8.new_workspace()
    a_q = torch.empty((m, k), dtype=torch.uint8, device="cuda")
    s_a = torch.empty(1, dtype=torch.float32, device="cuda")
    out = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    for _ in range(2):  # warm up outside the capture
        fp8.quant_dynamic(x, workspace=ws, q=a_q, scale=s_a)
        fp8.scaled_mm(a_q, w_q, s_a, s_w, True, out=out, accum=accum)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fp8.quant_dynamic(x, workspace=ws, q=a_q, scale=s_a)
        fp8.scaled_mm(a_q, w_q, s_a, s_w, True, out=out, accum=accum)
    torch.cuda.synchronize()

    ref = _eager(x, w_q, s_w, ws, accum)
    x2 = dev_bf16(synth.activations(8, m, k, outliers=False, scale=3.0))
    ref2 = _eager(x2, w_q, s_w, ws, accum)
    for rep in range(4):
        a_q.zero_(); s_a.zero_(); out.zero_()
        if rep == 2:
            x.copy_(x2)           # the graph reads whatever the buffer holds
        want = ref2 if rep >= 2 else ref
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(a_q, want[0]), rep
        assert torch.equal(s_a, want[1]), rep
        assert torch.equal(out.view(torch.int16), want[2].view(torch.int16)), rep
