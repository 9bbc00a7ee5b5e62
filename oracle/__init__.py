"""CPU oracle for the FP8 W8A8 linear layer: TEST INFRASTRUCTURE ONLY.

This package is the slow, obviously-correct reference the HIP path is checked
against.  Only the test-suite, the smoke check and the benchmark's CPU-baseline
leg may import it; the product library never does and has no CPU fallback.
It shares no code with the HIP path: it reads bf16 bit patterns and e4m3fn
bytes produced by the seeded input generators and computes everything itself
in NumPy (fp32 where the method fixes fp32, exact fp64/int64 elsewhere).

Sources (page title, then the part of the page):
  * "Prototype FP8Linear W8A8 runtime quantization" (nm-vllm issue 190),
    opening post: weights and activations are quantized at run time to
    torch.float8_e4m3fn and multiplied by a W8A8 FP8 GEMM.
  * "Fp8 Quantization Support" (compressed-tensors PR 62), description and
    recipe: fp8 means float8_e4m3fn; float and int quantization differ in range
    and rounding; the scheme is symmetric with one scale per tensor.
  * "[Kernel] Implement fallback for FP8 channelwise using torch._scaled_mm"
    (vLLM PR 6552), description: a channelwise (per output channel) weight
    scale is applied as a rescale after a per-tensor scaled GEMM.

oracle.glue holds the steps between the linears of the chained-linears
workload (residual add, RMS normalization, gated activation), which the pages
do not define; its readings are stated there.

Every function is pinned by tests marked ``not gpu`` to facts fixed outside
itself (closed forms, the 256-pattern table, exhaustive bf16 sweeps, a library
cast, int64 brute force).  The end-to-end model quality numbers on the pages
need checkpoints and datasets that are not available: parity unpinned for
those, and for any multi-layer drift.
"""
from .e4m3 import E4M3_MAX, decode, encode, positive_grid  # noqa: F401
from . import e5m2  # noqa: F401
from .w8a8 import FORMATS  # noqa: F401
from .w8a8 import (  # noqa: F401
    bf16_bits_to_f32,
    amax,
    scale_from_amax,
    quant_static,
    quant_dynamic,
    quant_weight,
    gemm_exact,
    scaled_mm,
    dequant_row_norms,
    to_bf16_rne,
)
from .glue import (  # noqa: F401
    add_bf16,
    rmsnorm,
    silu_mul,
    f32_to_bf16_bits,
    f64_to_bf16_bits,
    bf16_ulp_distance,
)
