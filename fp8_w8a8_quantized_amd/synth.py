"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no arithmetic of the quantized linear itself: it only draws
random numbers and rounds them to bf16 with torch's CPU cast (round to nearest
even).  Everything downstream (scales, codes, GEMMs) is computed separately by
the HIP library and by the CPU oracle from these same bit patterns.

Recipe (every draw float32, then one RNE rounding to bf16):
  * activations  A ~ N(0, 1); optionally round(0.01 * K) "outlier" columns,
    drawn without replacement and shared by all rows, multiplied by 20 before
    the bf16 rounding;
  * weights      W ~ N(0, 0.02); optionally every row n multiplied by
    c_n = exp(U(ln 0.25, ln 4)) (log-uniform on [0.25, 4]) before rounding;
  * bias         b ~ N(0, 0.1).
Each tensor's generator is PCG64 seeded by SeedSequence([config, layer, role,
sub]), so any tensor can be regenerated on its own.

The shapes stand in for the pages' models (Llama-3-8B-Instruct and
Mistral-7B checkpoints, which are not available): they take the models'
linear-layer shapes only.
"""
import numpy as np
import torch

ROLE_A, ROLE_W, ROLE_C, ROLE_OUTLIER, ROLE_BIAS = 0, 1, 2, 3, 4

# Llama-3-8B decoder linears as (name, K, N): fused QKV, O, fused gate_up, down.
LLAMA3_8B_LINEARS = (
    ("qkv", 4096, 6144),
    ("o", 4096, 4096),
    ("gate_up", 4096, 28672),
    ("down", 14336, 4096),
)
# Mistral-7B-shaped linears with M in {1, 3, 7, 13} and N not a multiple of 16.
MISTRAL_7B_SKINNY_M = (1, 3, 7, 13)
MISTRAL_7B_KN = (
    (4096, 4096), (4096, 14336), (4096, 4100), (4096, 1030), (4096, 6144), (14336, 4096),
)


def generator(config, layer, role, sub=0):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([config, layer, role, sub])))


def f32_to_bf16_bits(x):
    """float32 array -> bf16 bit patterns (uint16), round to nearest even."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def activations(config, m, k, layer=0, sub=0, outliers=False, scale=1.0):
    """bf16 bits [m, k] ~ N(0, scale^2), optionally with 1% outlier columns x20."""
    x = generator(config, layer, ROLE_A, sub).standard_normal((m, k), dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    if outliers and k > 0:
        n_out = int(round(0.01 * k))
        idx = generator(config, layer, ROLE_OUTLIER, sub).choice(k, size=n_out, replace=False)
        x[:, idx] *= np.float32(20.0)
    return f32_to_bf16_bits(x)


def weights(config, n, k, layer=0, sub=0, row_multipliers=False, std=0.02):
    """bf16 bits [n, k] ~ N(0, std^2), optionally rows scaled by LogU(0.25, 4)."""
    w = generator(config, layer, ROLE_W, sub).standard_normal((n, k), dtype=np.float32)
    w *= np.float32(std)
    if row_multipliers:
        u = generator(config, layer, ROLE_C, sub).uniform(np.log(0.25), np.log(4.0), size=n)
        w *= np.exp(u).astype(np.float32)[:, None]
    return f32_to_bf16_bits(w)


def weights_device(config, n, k, layer=0, sub=0, row_multipliers=False, std=0.02, device="cuda"):
    """torch.bfloat16 [n, k] on `device`, the weights recipe drawn by torch's
    device generator (Philox) seeded from SeedSequence([config, layer, role,
    sub]): for stacks of many large layers, whose host draws would dominate
    set-up time.  The row multipliers come from the host generator above.
    Copy the result to the host to hand the same values to the oracle."""
    seed = int(np.random.SeedSequence([config, layer, ROLE_W, sub]).generate_state(1)[0])
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    w = torch.randn((n, k), generator=g, device=device, dtype=torch.float32)
    w *= std
    if row_multipliers:
        u = generator(config, layer, ROLE_C, sub).uniform(np.log(0.25), np.log(4.0), size=n)
        w *= torch.from_numpy(np.exp(u).astype(np.float32)).to(device)[:, None]
    return w.to(torch.bfloat16)


def bias(config, n, layer=0, sub=0, std=0.1):
    b = generator(config, layer, ROLE_BIAS, sub).standard_normal(n, dtype=np.float32)
    return f32_to_bf16_bits(b * np.float32(std))


def bf16_bits_to_torch(bits):
    """uint16 numpy bits -> torch.bfloat16 CPU tensor with the same bits."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
