"""A Llama-3-8B-shaped stack of W8A8 linears with the steps between them:
the chained-linears workload, run entirely through the library's calls.

Per layer, on the residual stream h (bf16 [M, 4096]); every linear's input is
re-quantized with a fresh dynamic per-tensor scale, and every linear has
channelwise weight scales:

    h  <- h + d_prev; (q, s) = quant(rmsnorm(h))     fp8_add_rmsnorm_quant_dynamic
    qkv = W8A8(q, W_qkv)                              fp8_scaled_mm   [M, 6144]
    (q, s) = quant(qkv[:, :4096])                     fp8_quant_dynamic (the Q slice
                                                      stands in for attention's output)
    o   = W8A8(q, W_o)                                fp8_scaled_mm   [M, 4096]
    h  <- h + o;     (q, s) = quant(rmsnorm(h))       fp8_add_rmsnorm_quant_dynamic
    gu  = W8A8(q, W_gate_up)                          fp8_scaled_mm   [M, 28672]
    (q, s) = quant(silu(gate) * up)                   fp8_silu_mul_quant_dynamic
    d   = W8A8(q, W_down)                             fp8_scaled_mm   [M, 4096]

The residual add of a layer's last output happens in the next layer's first
call (after the last layer, in a final one).  The block glue is not on the
pages; its definitions are readings (unit-weight RMS normalization with eps
1e-5, gate-first SiLU*mul, Q-slice attention stand-in).  Nothing here
allocates after set-up, so a whole pass can be captured into a HIP graph.
"""
import torch

import fp8_w8a8_quantized_amd as fp8
from fp8_w8a8_quantized_amd import synth

D_MODEL, D_QKV, D_FF = 4096, 6144, 14336
SHAPES = (("qkv", D_MODEL, D_QKV), ("o", D_MODEL, D_MODEL), ("gate_up", D_MODEL, 2 * D_FF), ("down", D_FF, D_MODEL))
EPS = 1e-5


class Chain:
    def __init__(self, layers=32, config=5, accum="fp32", device="cuda"):
        self.layers, self.config, self.accum, self.device = layers, config, accum, device
        self.w = []
        for layer in range(layers):
            per = []
            for sub, (name, k, n) in enumerate(SHAPES):
                wb = synth.weights_device(config, n, k, layer=layer, sub=sub, row_multipliers=True, device=device)
                per.append(fp8.quant_weight(wb, per_channel=True))
                del wb
            self.w.append(per)
        self._bufs = {}

    def weight_bf16(self, layer, sub):
        """The bf16 weights of one linear, regenerated (for checks)."""
        name, k, n = SHAPES[sub]
        return synth.weights_device(self.config, n, k, layer=layer, sub=sub, row_multipliers=True,
                                    device=self.device)

    def buffers(self, m):
        if m not in self._bufs:
            dev, bf = self.device, torch.bfloat16
            self._bufs[m] = dict(
                h=[torch.empty((m, D_MODEL), dtype=bf, device=dev) for _ in range(2)],
                qkv=torch.empty((m, D_QKV), dtype=bf, device=dev),
                o=torch.empty((m, D_MODEL), dtype=bf, device=dev),
                gu=torch.empty((m, 2 * D_FF), dtype=bf, device=dev),
                d=torch.empty((m, D_MODEL), dtype=bf, device=dev),
                out=torch.empty((m, D_MODEL), dtype=bf, device=dev),
                q=torch.empty((m, D_FF), dtype=torch.uint8, device=dev),
                s=torch.empty(1, dtype=torch.float32, device=dev),
                ws=fp8.norm_workspace(m, dev),
            )
        return self._bufs[m]

    def forward(self, x, out=None):
        """Run every layer on x (bf16 [M, 4096]); returns the final residual
        stream (bf16 [M, 4096], in `out` or a per-M buffer)."""
        m = x.shape[0]
        B = self.buffers(m)
        q, s, ws = B["q"], B["s"], B["ws"]
        h_cur, d_prev = x, None
        slot = 0
        for layer in range(self.layers):
            (wq_qkv, sw_qkv), (wq_o, sw_o), (wq_gu, sw_gu), (wq_d, sw_d) = self.w[layer]
            h_next = B["h"][slot]
            qa = q[:, :D_MODEL]
            if d_prev is None:
                fp8.add_rmsnorm_quant(h_cur, eps=EPS, q=qa, scale=s, workspace=ws)
            else:
                fp8.add_rmsnorm_quant(h_cur, d_prev, h_out=h_next, eps=EPS, q=qa, scale=s, workspace=ws)
                h_cur, slot = h_next, slot ^ 1
            fp8.scaled_mm(qa, wq_qkv, s, sw_qkv, True, out=B["qkv"], accum=self.accum)
            fp8.quant_dynamic(B["qkv"][:, :D_MODEL], workspace=ws, q=qa, scale=s)
            fp8.scaled_mm(qa, wq_o, s, sw_o, True, out=B["o"], accum=self.accum)
            h_next = B["h"][slot]
            fp8.add_rmsnorm_quant(h_cur, B["o"], h_out=h_next, eps=EPS, q=qa, scale=s, workspace=ws)
            h_cur, slot = h_next, slot ^ 1
            fp8.scaled_mm(qa, wq_gu, s, sw_gu, True, out=B["gu"], accum=self.accum)
            fp8.silu_mul_quant(B["gu"], q=q, scale=s, workspace=ws)
            fp8.scaled_mm(q, wq_d, s, sw_d, True, out=B["d"], accum=self.accum)
            d_prev = B["d"]
        out = B["out"] if out is None else out
        # the last layer's residual add (its normalization and codes are not used)
        fp8.add_rmsnorm_quant(h_cur, d_prev, h_out=out, eps=EPS, q=q[:, :D_MODEL], scale=s, workspace=ws)
        return out
