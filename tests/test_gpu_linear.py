"""The one-call W8A8 linear (fp8_linear_dynamic) on the GPU.

Codes and scale are bit-exact against the CPU oracle, the output is within
the GEMM tolerance of the oracle and bit-identical to the two-call path
(fp8_quant_dynamic, then fp8_scaled_mm)."""
import numpy as np
import pytest
import torch

import oracle
import fp8_w8a8_quantized_amd as fp8
from fp8_w8a8_quantized_amd import synth
from _helpers import say, dev_bf16, host_u8, host_f32, host_bf16_bits, assert_gemm_close

pytestmark = pytest.mark.gpu

def _weights(cfg, m, k, n, per_channel, rowmul=False, with_bias=False):
    w = synth.weights(cfg, n, k, row_multipliers=rowmul)
    b = synth.bias(cfg, n) if with_bias else None
    w_q, s_w = fp8.quant_weight(dev_bf16(w), per_channel)
    wq_ref, sw_ref = oracle.quant_weight(w, per_channel)
    torch.cuda.synchronize()
    assert np.array_equal(host_f32(s_w), sw_ref) and np.array_equal(host_u8(w_q), wq_ref)
    return dict(w_q=w_q, s_w=s_w, wq=wq_ref, sw=sw_ref, bias=dev_bf16(b) if b is not None else None, bias_bits=b)


def _check(x_bits, x_dev, d, per_channel, ws, out=None, a_q=None, s_a=None):
    out, a_q, s_a = fp8.linear_dynamic(x_dev, d["w_q"], d["s_w"], per_channel, d["bias"], workspace=ws,
                                       out=out, a_q=a_q, s_a=s_a)
    q2, s2 = fp8.quant_dynamic(x_dev)
    out2 = fp8.scaled_mm(q2, d["w_q"], s2, d["s_w"], per_channel, d["bias"])
    torch.cuda.synchronize()
    aq_ref, sa_ref = oracle.quant_dynamic(x_bits)
    assert host_f32(s_a)[0] == sa_ref, (host_f32(s_a)[0], sa_ref)
    assert np.array_equal(host_u8(a_q), aq_ref)
    ob = host_bf16_bits(out)
    assert np.array_equal(ob, host_bf16_bits(out2)), "differs from the two-call path"
    ref = oracle.scaled_mm(aq_ref, d["wq"], sa_ref, d["sw"], per_channel, d["bias_bits"])
    assert_gemm_close(ob, ref, aq_ref, sa_ref, d["wq"], d["sw"], per_channel, bias_bits=d["bias_bits"])
    return out


# the four decode linears of an 8B-class model (one-block, two-block and
# interleaved-K skinny kernels, plain and non-temporal weight loads), ragged
# M, N and K, M up to 64 (four row blocks of the skinny kernel) and an
# activation past the one-launch quantizer's size
@pytest.mark.parametrize("m,k,n,pc,bias", [
    (16, 4096, 6144, True, False), (16, 4096, 4096, False, False), (16, 4096, 28672, True, False),
    (16, 14336, 4096, True, True), (1, 4096, 4100, True, True), (3, 2048, 16392, False, False),
    (13, 1024, 16400, True, True), (7, 8192, 1030, True, False), (5, 16, 17, True, True),
    (64, 1024, 300, False, True), (33, 512, 4100, True, False), (64, 32768, 64, True, False)])
def test_linear_decode_shapes(m, k, n, pc, bias):
    say("linear decode", m, k, n, pc, bias)
    x = synth.activations(3, m, k, outliers=True)
    d = _weights(3, m, k, n, pc, rowmul=pc, with_bias=bias)
    ws = fp8.new_linear_workspace()
    _check(x, dev_bf16(x), d, pc, ws)


# M above 64 on a problem too small for the matrix-core tiles (skinny kernel,
# two grid rows) and above 256 (matrix-core GEMM), a large activation, a
# misaligned activation view (element-wise loads), K % 16 != 0 (byte-granular
# skinny kernel)
@pytest.mark.parametrize("case", ["m65", "m300", "big_act", "x_view", "k_ragged"])
def test_linear_other_shapes(case):
    say("linear other", case)
    m, k, n = {"m65": (65, 1024, 520), "m300": (300, 1024, 520), "big_act": (64, 32784, 64),
               "x_view": (16, 4096, 1030), "k_ragged": (9, 4100, 33)}[case]
    x = synth.activations(4, m, k + (1 if case == "x_view" else 0))
    xd = dev_bf16(x)
    if case == "x_view":
        x, xd = x[:, 1:].copy(), xd[:, 1:]   # base pointer 2 bytes past alignment
    d = _weights(4, m, k, n, True, with_bias=True)
    ws = fp8.new_linear_workspace()
    _check(x, xd, d, True, ws)


def test_linear_empty_problems():
    say("linear empty")
    d = _weights(5, 4, 64, 32, True)
    ws = fp8.new_linear_workspace()
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    out, a_q, s_a = fp8.linear_dynamic(x, d["w_q"], d["s_w"], True, workspace=ws)
    torch.cuda.synchronize()
    assert out.shape == (0, 32) and host_f32(s_a)[0] == 1.0
    # N == 0: the codes and the scale are still produced
    xb = synth.activations(5, 4, 64)
    w0 = torch.zeros((0, 64), dtype=torch.uint8, device="cuda")
    s0 = torch.zeros(0, dtype=torch.float32, device="cuda")   # one scale per (absent) output channel
    out, a_q, s_a = fp8.linear_dynamic(dev_bf16(xb), w0, s0, True, workspace=ws)
    aq_ref, sa_ref = oracle.quant_dynamic(xb)
    torch.cuda.synchronize()
    assert out.shape == (4, 0) and host_f32(s_a)[0] == sa_ref and np.array_equal(host_u8(a_q), aq_ref)


def test_linear_workspace_reused_across_shapes():
    """One workspace for calls of different shapes back to back (one- and
    two-launch quantization, every skinny kernel)."""
    ws = fp8.new_linear_workspace()
    for i, (m, k, n) in enumerate([(16, 4096, 6144), (3, 14336, 4096), (16, 4096, 28672), (1, 1024, 300),
                                   (16, 4096, 6144)]):
        say("linear reuse", i, m, k, n)
        x = synth.activations(10 + i, m, k, outliers=(i % 2 == 0))
        d = _weights(10 + i, m, k, n, True)
        _check(x, dev_bf16(x), d, True, ws)


def test_linear_graph_replays():
    """The call captured in a HIP graph and replayed with new activations
    copied in between (eager library calls and synchronizations between the
    replays): every replay equals the eager two-call result."""
    m, k, n = 16, 4096, 6144
    d = _weights(20, m, k, n, True, with_bias=True)
    ws = fp8.new_linear_workspace()
    xd = torch.empty((m, k), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    a_q = torch.empty((m, k), dtype=torch.uint8, device="cuda")
    s_a = torch.empty(1, dtype=torch.float32, device="cuda")
    xd.copy_(dev_bf16(synth.activations(20, m, k)))
    fp8.linear_dynamic(xd, d["w_q"], d["s_w"], True, d["bias"], workspace=ws, out=out, a_q=a_q, s_a=s_a)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fp8.linear_dynamic(xd, d["w_q"], d["s_w"], True, d["bias"], workspace=ws, out=out, a_q=a_q, s_a=s_a)
    torch.cuda.synchronize()
    for r in range(4):
        say("linear graph replay", r)
        x = synth.activations(21 + r, m, k, outliers=(r % 2 == 1), scale=[1.0, 3.0, 0.01, 1.0][r])
        xd.copy_(dev_bf16(x))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        q2, s2 = fp8.quant_dynamic(xd)
        out2 = fp8.scaled_mm(q2, d["w_q"], s2, d["s_w"], True, d["bias"])
        torch.cuda.synchronize()
        aq_ref, sa_ref = oracle.quant_dynamic(x)
        assert host_f32(s_a)[0] == sa_ref and np.array_equal(host_u8(a_q), aq_ref)
        assert np.array_equal(host_bf16_bits(out), host_bf16_bits(out2))


def test_concurrent_streams_with_their_own_workspaces():
    """Two streams run the whole linear back to back, eight calls each, with
    their own workspace, operands and outputs: a 300 x 4096 -> 1030
    activation (two-launch quantization, its per-block maxima in the
    workspace) beside the 16 x 14336 -> 4096 decode input.  Each stream
    also alternates between two inputs, so a stale maximum from another
    call would change a scale.  Every output, code and scale equals the
    same call made alone (and the oracle's codes and scale)."""
    cases = [(300, 4096, 1030, 30), (16, 14336, 4096, 40)]
    work = []
    for m, k, n, cfg in cases:
        d = _weights(cfg, m, k, n, True, rowmul=True, with_bias=True)
        xs = [synth.activations(cfg + j, m, k, outliers=(j == 0), scale=[1.0, 5.0][j]) for j in range(2)]
        xd = [dev_bf16(x) for x in xs]
        refs = []
        for j in range(2):
            out, a_q, s_a = fp8.linear_dynamic(xd[j], d["w_q"], d["s_w"], True, d["bias"],
                                               workspace=fp8.new_linear_workspace())
            torch.cuda.synchronize()
            aq_ref, sa_ref = oracle.quant_dynamic(xs[j])
            assert host_f32(s_a)[0] == sa_ref and np.array_equal(host_u8(a_q), aq_ref)
            refs.append((out.clone(), a_q.clone(), s_a.clone()))
        work.append(dict(d=d, xd=xd, refs=refs, ws=fp8.new_linear_workspace(), stream=torch.cuda.Stream()))
    torch.cuda.synchronize()
    results = [[] for _ in work]
    for it in range(8):
        for w, res in zip(work, results):
            with torch.cuda.stream(w["stream"]):
                out, a_q, s_a = fp8.linear_dynamic(w["xd"][it % 2], w["d"]["w_q"], w["d"]["s_w"], True,
                                                   w["d"]["bias"], workspace=w["ws"])
                res.append((it % 2, out, a_q, s_a))
    torch.cuda.synchronize()
    for (m, k, n, _), w, res in zip(cases, work, results):
        say("concurrent stream", m, k, n, len(res), "calls")
        for j, out, a_q, s_a in res:
            ref_out, ref_q, ref_s = w["refs"][j]
            assert torch.equal(s_a, ref_s) and torch.equal(a_q, ref_q)
            assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
