"""The chained-linears workload (a Llama-3-8B-shaped stack, see
fp8_w8a8_quantized_amd/chain.py) on the GPU.

What the oracle can check element by element from seeded inputs is the
first linear of a pass: its input is the seeded residual stream, so the
oracle recomputes the RMS normalization, the codes, the weight codes and the
exact GEMM itself.  Every later step's input is a GPU output; those steps are
covered one by one, from seeded inputs, by the producer, quantization and
GEMM tests.  The whole stack is also run by the oracle alone, from the same
seeded input and its own weight codes, and the GPU's last-layer outputs and
final residual stream are compared with that run within a relative bound
(never feeding GPU values to the oracle).  Here the stack is also checked for
determinism, finiteness and HIP-graph replay against eager execution.
"""
import numpy as np
import pytest
import torch

import oracle
import oracle.glue as glue
from fp8_w8a8_quantized_amd import chain, synth
from _helpers import say, dev_bf16, host_bf16_bits, assert_gemm_close

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def stack():
    say("building a 2-layer stack")
    c = chain.Chain(layers=2)
    torch.cuda.synchronize()
    return c


def _first_linear_check(c, m, rows):
    x_bits = synth.activations(5, m, chain.D_MODEL, layer=99, outliers=True)
    x = dev_bf16(x_bits)
    c.forward(x)
    torch.cuda.synchronize()
    # layer 1's QKV output overwrote layer 0's: rerun a one-layer view of the stack
    one = chain.Chain.__new__(chain.Chain)
    one.__dict__.update(c.__dict__)
    one.layers, one._bufs = 1, {}
    one.forward(x)
    torch.cuda.synchronize()
    qkv_gpu = host_bf16_bits(one.buffers(m)["qkv"])[rows]
    y = oracle.rmsnorm(x_bits, chain.EPS)
    aq, sa = oracle.quant_dynamic(y)
    w_bits = host_bf16_bits(c.weight_bf16(0, 0))
    wq, sw = oracle.quant_weight(w_bits, True)
    ref = oracle.scaled_mm(aq[rows], wq, sa, sw, True)
    assert_gemm_close(qkv_gpu, ref, aq[rows], sa, wq, sw, True)


def test_first_linear_decode_matches_oracle(stack):
    say("first linear, M = 16")
    _first_linear_check(stack, 16, np.arange(16))


def test_first_linear_prefill_matches_oracle(stack):
    m = 16 * 1024
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([rng.choice(m, 48, replace=False), np.arange(m - 16, m)]))
    say("first linear, M = 16384, sampled rows", len(rows))
    _first_linear_check(stack, m, rows)


@pytest.fixture(scope="module")
def oracle_weights(stack):
    """The oracle's own weight codes and channel scales for every linear of
    the stack, from the same seeded bf16 weights."""
    out = []
    for layer in range(stack.layers):
        per = []
        for sub, (name, k, n) in enumerate(chain.SHAPES):
            per.append(oracle.quant_weight(host_bf16_bits(stack.weight_bf16(layer, sub)), True))
            say(f"oracle weight codes: layer {layer} {name}")
        out.append(per)
    return out


def _oracle_stack(x_bits, wq):
    """The stack of chain.py computed by the oracle alone: per layer, the
    residual add and RMS normalization of the block glue, a fresh dynamic
    per-tensor quantization before every linear, the exact scaled GEMMs with
    channel scales rounded once to bf16, the Q slice of the QKV output as the
    attention stand-in, and gate-first SiLU*mul; after the last layer, its
    residual add.  Returns the final residual stream and the last layer's
    linear outputs (bf16 bits)."""
    def linear(bits, w):
        a_q, s_a = oracle.quant_dynamic(bits)
        return glue.f64_to_bf16_bits(oracle.scaled_mm(a_q, w[0], s_a, w[1], True))

    h, d, last = x_bits, None, {}
    for per in wq:
        if d is not None:
            h = glue.add_bf16(h, d)
        qkv = linear(glue.rmsnorm(h, chain.EPS), per[0])
        o = linear(qkv[:, :chain.D_MODEL], per[1])
        h = glue.add_bf16(h, o)
        gu = linear(glue.rmsnorm(h, chain.EPS), per[2])
        d = linear(glue.silu_mul(gu, chain.D_FF), per[3])
        last = dict(qkv=qkv, o=o, gu=gu, d=d)
    return glue.add_bf16(h, d), last


def _rel_l2(gpu_bits, ref_bits):
    g = oracle.bf16_bits_to_f32(gpu_bits).astype(np.float64)
    r = oracle.bf16_bits_to_f32(ref_bits).astype(np.float64)
    return float(np.linalg.norm(g - r) / np.linalg.norm(r))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("m", [16, 96])
def test_stack_against_an_oracle_run_of_the_whole_stack(stack, oracle_weights, m):
    """The GPU stack against the oracle's own run of it (M = 16: the skinny
    GEMMs; M = 96: the skinny kernel in two grid rows of M for QKV, O and
    down, and the matrix-core GEMM for gate_up, on the pitched code slices).

    Nothing of the GPU's enters the oracle's run, so the two drift apart
    where rounding differs.  With the same codes on both sides an output
    differs from the oracle's rounding of the exact sum by at most one bf16
    step, and only where the float32 sum lands across a rounding midpoint.
    Such a step can move a later code by one e4m3 step, or (when it hits a
    tensor's largest value) that tensor's scale by one bf16 step, which
    moves the codes near their rounding midpoints.  Each keeps the relative
    error at a fraction of one e4m3 step (2^-4) spread over few terms.  A
    wiring mistake (a wrong buffer, slot, slice or layer's weights, or a
    missing residual add) changes the result by order one.  Bound: relative
    L2 error at most 2^-5 for the last layer's four linear outputs and the
    final residual stream.
    """
    x_bits = synth.activations(5, m, chain.D_MODEL, layer=97, outliers=True)
    out = stack.forward(dev_bf16(x_bits)).clone()
    torch.cuda.synchronize()
    B = stack.buffers(m)
    gpu = {name: host_bf16_bits(B[name]) for name in ("qkv", "o", "gu", "d")}
    gpu["h"] = host_bf16_bits(out)
    say(f"oracle stack run, M = {m}")
    h_ref, last = _oracle_stack(x_bits, oracle_weights)
    ref = dict(last, h=h_ref)
    for name in ("qkv", "o", "gu", "d", "h"):
        rel = _rel_l2(gpu[name], ref[name])
        same = float(np.mean(gpu[name] == ref[name]))
        g = oracle.bf16_bits_to_f32(gpu[name]).astype(np.float64)
        r = oracle.bf16_bits_to_f32(ref[name]).astype(np.float64)
        worst = float(np.max(np.abs(g - r)) / np.sqrt(np.mean(r * r)))
        say(f"  {name}: relative L2 {rel:.3e}, bit-identical {same:.4f}, largest difference {worst:.3e} x rms")
        assert rel <= 2.0 ** -5, (name, rel)


def test_stack_deterministic_finite_and_graph_replay(stack):
    prompts, seq = 16, 64
    x = dev_bf16(synth.activations(5, prompts * seq, chain.D_MODEL, layer=98, outliers=True))
    say("prefill", tuple(x.shape))
    h = stack.forward(x).clone()
    h2 = stack.forward(x).clone()
    torch.cuda.synchronize()
    assert torch.equal(h, h2)
    assert torch.isfinite(h.float()).all()
    start = h[seq - 1::seq].contiguous()          # last token of each prompt
    assert start.shape == (prompts, chain.D_MODEL)

    def eager(steps):
        cur = start.clone()
        outs = []
        for _ in range(steps):
            cur = stack.forward(cur).clone()
            outs.append(cur)
        return outs

    ref = eager(4)
    torch.cuda.synchronize()
    for o in ref:
        assert torch.isfinite(o.float()).all()
    # one captured decode step, replayed with its output fed back to its input
    xin = start.clone()
    xout = torch.empty_like(xin)
    stack.forward(xin, out=xout)                  # buffers exist before capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        stack.forward(xin, out=xout)
        xin.copy_(xout)
    xin.copy_(start)
    torch.cuda.synchronize()
    for t in range(4):
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(xout, ref[t]), t
