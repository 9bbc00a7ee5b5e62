"""The Python binding checks every tensor before it calls the library.

The kernels trust the sizes they are given: a per-channel scale vector
shorter than N, a bias of the wrong length, an output of the wrong shape, a
host tensor or a workspace that is too small would become out-of-range
device accesses.  These tests run on the host only: device tensors are
stood in for by CPU tensors (the device predicate is patched to accept
them) and the library is replaced by a stub that fails the test if any
function is called, so each case must be rejected before a C call.
"""
import pytest
import torch

import fp8_w8a8_quantized_amd as fp8


class _NoCalls:
    def __getattr__(self, name):
        raise AssertionError(f"library function {name} called despite invalid arguments")


class _SizesOnly:
    """Answers the workspace-size queries the binding makes; fails on anything else."""
    def fp8_quant_workspace_bytes(self):
        return 4096

    def fp8_linear_workspace_bytes(self):
        return 4096

    def fp8_norm_quant_workspace_bytes(self, rows):
        return 4096 + 8 * rows

    def __getattr__(self, name):
        raise AssertionError(f"library function {name} called despite invalid arguments")


@pytest.fixture
def host_tensors(monkeypatch):
    """Let CPU tensors pass the device check; forbid library calls."""
    monkeypatch.setattr(fp8, "_on_gpu", lambda t: True)
    monkeypatch.setattr(fp8, "lib", lambda: _SizesOnly())


def _gemm(M=4, N=32, K=64, per_channel=True):
    return dict(a_q=torch.zeros((M, K), dtype=torch.uint8), w_q=torch.zeros((N, K), dtype=torch.uint8),
                s_a=torch.ones(1, dtype=torch.float32),
                s_w=torch.ones(N if per_channel else 1, dtype=torch.float32), per_channel=per_channel)


def _mm(**over):
    d = _gemm()
    d.update(over)
    return fp8.scaled_mm(d["a_q"], d["w_q"], d["s_a"], d["s_w"], d["per_channel"], d.get("bias"),
                         out=d.get("out"), accum=d.get("accum", "fp32"))


def test_host_tensors_are_rejected(monkeypatch):
    monkeypatch.setattr(fp8, "lib", lambda: _NoCalls())
    d = _gemm()
    with pytest.raises(ValueError, match="device tensor"):
        fp8.scaled_mm(d["a_q"], d["w_q"], d["s_a"], d["s_w"], True)


@pytest.mark.parametrize("case,match", [
    (dict(s_w=torch.ones(1, dtype=torch.float32)), "s_w must have 32"),          # per-channel, 1 scale
    (dict(s_w=torch.ones(31, dtype=torch.float32)), "s_w must have 32"),
    (dict(s_w=torch.ones(32, dtype=torch.float64)), "s_w must be torch.float32"),
    (dict(s_a=torch.ones(2, dtype=torch.float32)), "s_a must have 1"),
    (dict(s_a=torch.ones(1, dtype=torch.bfloat16)), "s_a must be torch.float32"),
    (dict(bias=torch.zeros(31, dtype=torch.bfloat16)), "bias must have 32"),
    (dict(bias=torch.zeros(32, dtype=torch.float32)), "bias must be torch.bfloat16"),
    (dict(out=torch.empty((4, 31), dtype=torch.bfloat16)), "out must have shape"),
    (dict(out=torch.empty((4, 32), dtype=torch.float32)), "out must be torch.bfloat16"),
    (dict(out=torch.empty((32, 4), dtype=torch.bfloat16).t()), "unit column stride"),
    (dict(w_q=torch.zeros((32, 63), dtype=torch.uint8)), "K mismatch"),
    (dict(a_q=torch.zeros((4, 64), dtype=torch.int8)), "a_q must be torch.uint8"),
    (dict(accum="bf16"), "accumulation mode"),
])
def test_scaled_mm_rejects_bad_tensors(host_tensors, case, match):
    with pytest.raises(ValueError, match=match):
        _mm(**case)


def test_per_tensor_scale_must_be_one_element(host_tensors):
    d = _gemm(per_channel=False)
    with pytest.raises(ValueError, match="s_w must have 1"):
        fp8.scaled_mm(d["a_q"], d["w_q"], d["s_a"], torch.ones(32, dtype=torch.float32), False)


def test_quantizers_reject_bad_outputs_and_workspace(host_tensors):
    x = torch.zeros((4, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="workspace holds 64 bytes"):
        fp8.quant_dynamic(x, workspace=torch.empty(64, dtype=torch.uint8))
    with pytest.raises(ValueError, match="q must have shape"):
        fp8.quant_dynamic(x, q=torch.empty((4, 63), dtype=torch.uint8))
    with pytest.raises(ValueError, match="scale must have 1"):
        fp8.quant_dynamic(x, scale=torch.empty(2, dtype=torch.float32))
    with pytest.raises(ValueError, match="unknown fp8 format"):
        fp8.quant_dynamic(x, fmt="e3m4")
    with pytest.raises(ValueError, match="scale must be torch.float32"):
        fp8.quant_static(x, torch.ones(1, dtype=torch.float64))
    with pytest.raises(ValueError, match="scales must have 4"):
        fp8.quant_dynamic_per_row(x, scales=torch.empty(3, dtype=torch.float32))


def test_linear_and_producers_reject_bad_tensors(host_tensors):
    x = torch.zeros((4, 64), dtype=torch.bfloat16)
    d = _gemm()
    with pytest.raises(ValueError, match="s_w must have 32"):
        fp8.linear_dynamic(x, d["w_q"], torch.ones(1, dtype=torch.float32), True)
    with pytest.raises(ValueError, match="a_q must have shape"):
        fp8.linear_dynamic(x, d["w_q"], d["s_w"], True, a_q=torch.empty((4, 32), dtype=torch.uint8))
    with pytest.raises(ValueError, match="workspace holds"):
        fp8.linear_dynamic(x, d["w_q"], d["s_w"], True, workspace=torch.empty(16, dtype=torch.uint8))
    h = torch.zeros((16, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="workspace holds 4096 bytes, needs 4224"):
        # a plain quantizer workspace lacks room for the rows' statistics
        fp8.add_rmsnorm_quant(h, workspace=torch.empty(4096, dtype=torch.uint8))
    with pytest.raises(ValueError, match="delta must have shape"):
        fp8.add_rmsnorm_quant(h, delta=torch.zeros((16, 32), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="y_out must have shape"):
        fp8.silu_mul_quant(torch.zeros((4, 64), dtype=torch.bfloat16), y_out=torch.empty((4, 64), dtype=torch.bfloat16))
