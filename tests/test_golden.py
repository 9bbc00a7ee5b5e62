"""Pins from numbers printed on the pages (fixtures under tests/golden/)."""
import json
import os

import numpy as np

import oracle
from fp8_w8a8_quantized_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

MISTRAL_LAYER_LINEARS = [(4096, 4096), (1024, 4096), (1024, 4096), (4096, 4096),
                         (14336, 4096), (14336, 4096), (4096, 14336)]


def test_weight_memory_saving_is_one_byte_per_linear_weight():
    """bf16 -> fp8 saves exactly one byte per linear weight (no padding).

    The loader printed 13.4976 and 6.9976 for the same model; everything that
    is not a linear weight is identical in both runs, so the difference is
    sum(N*K) * (2 - bytes per quantized weight) over the linears.
    """
    g = json.load(open(os.path.join(GOLDEN, "mistral7b_weight_memory.json")))
    # bytes per quantized weight, as the oracle stores a linear's weight
    w = synth.weights(9, 48, 80)
    q, s = oracle.quant_weight(w, per_channel=False)
    per_weight = q.nbytes / (48 * 80)
    assert per_weight == 1.0
    n_linear = 32 * sum(n * k for n, k in MISTRAL_LAYER_LINEARS)
    saving_gib = n_linear * (2 - per_weight) / 2 ** 30
    printed = g["bf16_weights_gib"] - g["fp8_weights_gib"]
    assert abs(saving_gib - printed) < 5e-4, (saving_gib, printed)
