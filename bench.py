"""Benchmark of the FP8 W8A8 linear layer on one MI355X.

One step = the whole hot path over one batch: for each of the four linears
of a Llama-3-8B decoder layer (fused QKV 4096->6144, O 4096->4096, fused
gate_up 4096->28672, down 14336->4096), dynamic per-tensor quantization of
the bf16 activations, then the scaled FP8 GEMM with channelwise weight
scales and the rescale fused into its bf16 store.

Workloads (synthetic, seeded; the models' shapes only -- no checkpoints):
  decode   M = 16 tokens.  HBM-bound: reported in GB/s of algorithmic bytes.
           The weights rotate through 8 distinct copies of the layer
           (1.75 GB, several times the 256 MB Infinity Cache), as successive
           layers of a model would, so they stream from HBM.
  prefill  M = 16 x 1024 = 16384 tokens.  Matrix-core bound: TFLOP/s.
  skinny   single per-tensor linears at small M: 16 x 4096 -> 4096, and
           Mistral-7B-shaped GEMMs at M in {1, 3, 7, 13} (and 32, 64) with
           N not a multiple of 16, weights rotated over >= 1 GiB per shape.
  mid_m    the four Llama-3-8B GEMMs at M in {32, 64, 65, 128, 256, 512, 1024},
           between decode and prefill.

The default run (--workload all) prints the decode line (the headline value
and roofline) with a "prefill" object (both accumulation modes, per shape)
and "skinny", "mid_m" and "next" objects added, so one line carries both
halves of the metric.

Each step is captured once into a HIP graph and replayed (as a serving
loop would); --eager launches every kernel from Python instead.

Prints ONE JSON line.  The roofline object describes the dominant kernel
(the GEMM): algorithmic bytes (decode) or flops (prefill) per launch over
the mean launch time, measured with HIP events around graphs of
back-to-back GEMM launches; the cpu_baseline object times the CPU oracle on
a bounded sample of the same workload.
"""
import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import fp8_w8a8_quantized_amd as fp8  # noqa: E402
from fp8_w8a8_quantized_amd import synth  # noqa: E402

METRIC = "W8A8 scaled-GEMM TFLOP/s (% FP8 MFMA peak); decode M≤16 GB/s (% HBM peak)"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
FP8_PEAK_TFLOPS = 5000.0     # MI355X dense FP8 matrix throughput, published
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 matrix throughput, published
ROTATE_DECODE = 8
ROTATE_MIN_BYTES = 1 << 30   # skinny GEMMs: weights rotated over at least this many bytes
PREFILL_M = 16384
MID_M = (32, 64, 65, 128, 256, 512, 1024)


def quant_bytes(m, k):
    """Algorithmic HBM bytes of dynamic quantization: read bf16, write codes + scale."""
    return 2 * m * k + m * k + 4


def gemm_bytes(m, k, n, per_channel=True):
    """Algorithmic HBM bytes of the scaled GEMM: W and A codes once, bf16 out, scales."""
    return n * k + m * k + 2 * m * n + (4 * n if per_channel else 4) + 4


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def recorded_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed PMC record (profiles/traffic.json).

    The record holds FETCH_SIZE / WRITE_SIZE per shape, scaled by what the same
    counters read for a 1 GiB device copy, and the SHA-256 of the kernel's
    source when the counters were taken.  Returns the mean over the four
    shapes, or None when there is no record or the source has changed since.
    """
    import hashlib
    try:
        with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
            rec = json.load(f)["kernels"][kernel]
        with open(os.path.join(ROOT, rec["source"]), "rb") as f:
            if hashlib.sha256(f.read()).hexdigest() != rec["source_sha256"]:
                return None
        return int(round(rec["mean_traffic_bytes"]))
    except (OSError, KeyError, ValueError):
        return None


def build_layer(m, rotate, cfg=2, weights_from=None):
    """Quantized weights (on the GPU, per channel) and bf16 activations.

    cfg selects the activations' seed stream (2: decode, 3: prefill); the
    weights are the decode layer's (cfg 2) in both, or the first copy of
    `weights_from`'s when given (the same four shapes and channelwise scales).
    """
    lin = []
    for sub, (name, k, n) in enumerate(synth.LLAMA3_8B_LINEARS):
        if weights_from is not None:
            w_q, s_w = weights_from[sub]["copies"][0]
        else:
            w = synth.bf16_bits_to_torch(synth.weights(2, n, k, sub=sub, row_multipliers=True)).cuda()
            w_q, s_w = fp8.quant_weight(w, per_channel=True)
            del w
        copies = [(w_q, s_w)] + [(w_q.clone(), s_w.clone()) for _ in range(rotate - 1)]
        x = synth.bf16_bits_to_torch(synth.activations(cfg, m, k, sub=sub, outliers=True)).cuda()
        lin.append(dict(name=name, k=k, n=n, x=x, copies=copies,
                        a_q=torch.empty((m, k), dtype=torch.uint8, device="cuda"),
                        s_a=torch.empty(1, dtype=torch.float32, device="cuda"),
                        out=torch.empty((m, n), dtype=torch.bfloat16, device="cuda")))
    torch.cuda.synchronize()
    return lin


def run_step(lin, it, ws, accum):
    for L in lin:
        w_q, s_w = L["copies"][it % len(L["copies"])]
        fp8.quant_dynamic(L["x"], workspace=ws, q=L["a_q"], scale=L["s_a"])
        fp8.scaled_mm(L["a_q"], w_q, L["s_a"], s_w, True, out=L["out"], accum=accum)


def time_graph_per_launch(launch, n_launches, replays=3, windows=1):
    """Mean time per launch of a graph holding n_launches back-to-back calls
    made by launch(); HIP events on the stream the launches run on.  With
    windows > 1 the timed replays are repeated in that many windows and the
    median window's mean is returned (one slow window, e.g. a clock change
    right after other work, does not decide the figure)."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        launch()
    g.replay()
    torch.cuda.synchronize()
    means = []
    for _ in range(windows):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(replays):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        means.append(e0.elapsed_time(e1) * 1e-3 / (replays * n_launches))
    return float(np.median(means))


def time_eager_per_launch(launch, n_launches):
    """Mean time per launch of n_launches calls made by launch() from Python
    (one untimed pass first); HIP events on the launch stream."""
    launch()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    launch()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / n_launches


def copy_calibration(mib):
    """A fill, a device copy (3 times) and a sum over a buffer of `mib` MiB:
    kernels of known traffic, against which profiler byte counters are scaled."""
    nb = mib << 20
    src = torch.ones(nb, dtype=torch.uint8, device="cuda")   # fill: writes nb bytes
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)                                         # copy: reads and writes nb
    total = src.view(torch.int32).sum()                        # reduction: reads nb
    torch.cuda.synchronize()
    del src, dst, total


def time_steps(lin, ws, accum, steps, warmup, eager=False):
    """Wall time per step: each step's launches captured once per weight copy
    into a HIP graph and replayed (or launched eagerly)."""
    rotate = len(lin[0]["copies"])
    for i in range(warmup):
        run_step(lin, i, ws, accum)
    torch.cuda.synchronize()
    if eager:
        def step_fn(i):
            run_step(lin, i, ws, accum)
    else:
        # one HIP graph per weight copy; the library calls allocate nothing and
        # never synchronize, so a whole step (8 launches) replays as one graph
        step_graphs = []
        for r in range(rotate):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                run_step(lin, r, ws, accum)
            step_graphs.append(g)
        torch.cuda.synchronize()

        def step_fn(i):
            step_graphs[i % rotate].replay()
        for i in range(warmup):
            step_fn(i)
        torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step_fn(i)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def gemm_times(lin, accum, reps, windows=5):
    """Per-launch GEMM time of each linear: a graph of back-to-back GEMM
    launches over the weight copies (the activation codes and scale from the
    last step), timed in `windows` windows of 3 replays (the median window)."""
    out = []
    for L in lin:
        rotate = len(L["copies"])

        def launch(L=L):
            for _ in range(reps):
                for (w_q, s_w) in L["copies"]:
                    fp8.scaled_mm(L["a_q"], w_q, L["s_a"], s_w, True, out=L["out"], accum=accum)
        out.append(time_graph_per_launch(launch, reps * rotate, windows=windows))
    return out


def bench_prefill_modes(weights_from, args):
    """The four linears at M = 16384, in both accumulation modes: per-shape
    GEMM time, TFLOP/s and share of peak, and the whole step (quantization +
    GEMM for the four linears)."""
    m = PREFILL_M
    log(f"building inputs: prefill, M={m}")
    lin = build_layer(m, 1, cfg=3, weights_from=weights_from)
    ws = fp8.new_workspace()
    flops = [2 * m * L["k"] * L["n"] for L in lin]
    res = {"M": m, "workload": "llama3-8b prefill linears (qkv, o, gate_up, down), M=16384 (16 x 1024 tokens), "
                               "channelwise weight scales, dynamic per-tensor activation scale",
           "peak_tflops": {"fp8": FP8_PEAK_TFLOPS, "bf16": BF16_PEAK_TFLOPS}, "modes": {}}
    for accum in ("fp32", "fp8"):
        step_ms = time_steps(lin, ws, accum, steps=args.prefill_steps, warmup=2)
        per = gemm_times(lin, accum, reps=3)
        gemm_tflops = sum(flops) / sum(per) / 1e12
        r = {"kernel": f"gemm_mfma_kernel<4, {'true' if accum == 'fp32' else 'false'}, true, 0, 0>",
             "sums": ("bf16 matrix cores on exactly converted e4m3 values (fp32-class sums; the default)"
                      if accum == "fp32" else "fp8 matrix cores (13-bit sums inside each group of 8 products)"),
             "per_shape_us": {L["name"]: round(t * 1e6, 2) for L, t in zip(lin, per)},
             "per_shape_tflops": {L["name"]: round(f / t / 1e12, 1) for L, f, t in zip(lin, flops, per)},
             "gemm_tflops": round(gemm_tflops, 1),
             "frac_fp8_peak": round(gemm_tflops / FP8_PEAK_TFLOPS, 4),
             "step_ms": round(step_ms, 4),
             "step_tflops": round(sum(flops) / (step_ms * 1e-3) / 1e12, 1)}
        if accum == "fp32":
            r["frac_bf16_peak"] = round(gemm_tflops / BF16_PEAK_TFLOPS, 4)
        r["traffic"] = recorded_traffic(r["kernel"])
        res["modes"][accum] = r
        log(f"prefill {accum}: GEMM {gemm_tflops:.0f} TFLOP/s, step {step_ms:.3f} ms")
    del lin
    torch.cuda.empty_cache()
    return res


def bench_skinny(args):
    """Single per-tensor linears at small M (GEMM only; activations quantized
    once): 16 x 4096 -> 4096, and Mistral-7B-shaped GEMMs at M in {1, 3, 7,
    13} with N in {4096, 14336, 4100, 1030, 6144} (K = 4096) and 14336 -> 4096,
    plus M = 32 and 64 on the same shapes.  Each shape's weight rotates over
    copies totalling at least 1 GiB, so it streams from HBM.  A graph of one
    launch per copy is timed (with --eager: the launches from Python, one
    untimed pass first)."""
    log("building inputs: skinny GEMMs")
    pool = {}
    for j, (k, n) in enumerate(synth.MISTRAL_7B_KN):
        w = synth.bf16_bits_to_torch(synth.weights(4, n, k, sub=j)).cuda()
        w_q, s_w = fp8.quant_weight(w, per_channel=False)
        del w
        copies = -(-ROTATE_MIN_BYTES // (n * k))
        pool[(k, n)] = [(w_q, s_w)] + [(w_q.clone(), s_w) for _ in range(copies - 1)]
    torch.cuda.synchronize()
    cases = [(1, 16, 4096, 4096, "single linear 16x4096x4096, per tensor")]
    cases += [(4, m, k, n, "mistral-7b shapes, per tensor") for m in synth.MISTRAL_7B_SKINNY_M
              for (k, n) in synth.MISTRAL_7B_KN]
    cases += [(4, m, k, n, "mistral-7b shapes at larger M, per tensor") for m in (32, 64)
              for (k, n) in synth.MISTRAL_7B_KN]
    rows = []
    for (cfg, m, k, n, what) in cases:
        copies = pool[(k, n)]
        x = synth.bf16_bits_to_torch(synth.activations(cfg, m, k, sub=1000 + m)).cuda()
        a_q, s_a = fp8.quant_dynamic(x)
        out = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")

        def launch(copies=copies, a_q=a_q, s_a=s_a, out=out):
            for (w_q, s_w) in copies:
                fp8.scaled_mm(a_q, w_q, s_a, s_w, False, out=out)
        if args.eager:
            t = time_eager_per_launch(launch, len(copies))
        else:
            t = time_graph_per_launch(launch, len(copies))
        b = gemm_bytes(m, k, n, per_channel=False)
        rows.append({"M": m, "K": k, "N": n, "what": what, "us": round(t * 1e6, 2),
                     "GBps": round(b / t / 1e9, 1), "frac_hbm": round(b / t / 1e9 / HBM_PEAK_GBS, 4),
                     "algorithmic_bytes": b, "rotation_copies": len(copies)})
    del pool
    torch.cuda.empty_cache()
    hbm = [r for r in rows if r["M"] <= 16]
    return {"workload": "per-tensor W8A8 GEMMs at small M (decode), weights rotated over >= 1 GiB per shape; "
                        "bytes = N*K + M*K + 2*M*N + 8",
            "gemms": rows,
            "mean_frac_hbm_m_le_16": round(float(np.mean([r["frac_hbm"] for r in hbm])), 4)}


def bench_mid_m(args):
    """GEMMs between decode and prefill: M in {32, 64, 65, 128, 256, 512, 1024} rows
    on the Llama-3-8B shapes (channelwise scales, fp32-class sums), each
    weight rotated over copies totalling at least 1 GiB.  The call gives
    problems too small for the matrix-core tiles to the skinny kernel and
    runs 128 x 128 tiles where 256 x 256 ones are too few.  A graph of one
    launch per copy is timed; per GEMM: us, TFLOP/s, and GB/s of N*K + M*K +
    2*M*N + 4*N + 4 bytes."""
    log("building inputs: mid-M GEMMs")
    rows = []
    for sub, (name, k, n) in enumerate(synth.LLAMA3_8B_LINEARS):
        w = synth.bf16_bits_to_torch(synth.weights(5, n, k, sub=sub, row_multipliers=True)).cuda()
        w_q, s_w = fp8.quant_weight(w, per_channel=True)
        del w
        copies = [(w_q, s_w)] + [(w_q.clone(), s_w) for _ in range(-(-ROTATE_MIN_BYTES // (n * k)) - 1)]
        torch.cuda.synchronize()
        for m in MID_M:
            x = synth.bf16_bits_to_torch(synth.activations(5, m, k, sub=3000 + m, outliers=True)).cuda()
            a_q, s_a = fp8.quant_dynamic(x)
            out = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")

            def launch(copies=copies, a_q=a_q, s_a=s_a, out=out):
                for (wq, sw) in copies:
                    fp8.scaled_mm(a_q, wq, s_a, sw, True, out=out)
            t = time_eager_per_launch(launch, len(copies)) if args.eager else time_graph_per_launch(launch, len(copies))
            b = gemm_bytes(m, k, n)
            rows.append({"name": name, "M": m, "K": k, "N": n, "us": round(t * 1e6, 2),
                         "TFLOPs": round(2 * m * n * k / t / 1e12, 1), "GBps": round(b / t / 1e9, 1),
                         "rotation_copies": len(copies)})
        del copies, w_q
        torch.cuda.empty_cache()
    return {"workload": "llama3-8b linears at M = 32, 64, 65, 128, 256, 512, 1024 (between decode and prefill), channelwise weight "
                        "scales, fp32-class sums, weights rotated over >= 1 GiB per shape",
            "gemms": rows}


def bench_next(args):
    """The calls beyond the headline path, each timed like the GEMMs (a graph
    of back-to-back calls, the median of five timed windows): the
    producer-fused quantizations (residual add + RMS norm, SiLU*mul), the
    static activation quantization and the weight quantization on the device,
    at decode and prefill sizes of the Llama-3-8B layer; and e5m2 GEMMs (e5m2
    activations and weights, channelwise, exact sums), at decode size with
    weights rotated over 8 copies and at prefill size."""
    log("building inputs: next rows")
    bf = lambda bits: synth.bf16_bits_to_torch(bits).cuda()
    dev = "cuda"
    calls = []

    def timed(fn, n):
        def launch():
            for _ in range(n):
                fn()
        return time_graph_per_launch(launch, n, windows=5)

    def hbm_row(call, m, k, t, b, extra=None):
        r = {"call": call, "M": m, "K": k, "us": round(t * 1e6, 2), "GBps": round(b / t / 1e9, 1),
             "frac_hbm": round(b / t / 1e9 / HBM_PEAK_GBS, 4), "algorithmic_bytes": int(b)}
        r.update(extra or {})
        calls.append(r)

    d_ff = 14336
    for m in (16, PREFILL_M):
        n = 16 if m == 16 else 2
        h, d = bf(synth.activations(2, m, 4096, layer=7, outliers=True)), bf(synth.activations(2, m, 4096, layer=8))
        ho = torch.empty_like(h)
        q = torch.empty((m, d_ff), dtype=torch.uint8, device=dev)
        s = torch.empty(1, dtype=torch.float32, device=dev)
        nws = fp8.norm_workspace(m, dev)
        qa = q[:, :4096]
        t = timed(lambda: fp8.add_rmsnorm_quant(h, d, h_out=ho, q=qa, scale=s, workspace=nws), n)
        hbm_row("add_rmsnorm_quant (bf16 h + delta in, h' and e4m3 codes out)", m, 4096, t, m * 4096 * 7 + 4)
        sc = torch.tensor([0.05], dtype=torch.float32, device=dev)
        t = timed(lambda: fp8.quant_static(h, sc, q=qa), n)
        hbm_row("quant_static (bf16 in, e4m3 codes out)", m, 4096, t, m * 4096 * 3)
        del h, d, ho
        gu = bf(synth.activations(2, m, 2 * d_ff, layer=9, outliers=True))
        ws = fp8.new_workspace(dev)
        t = timed(lambda: fp8.silu_mul_quant(gu, q=q, scale=s, workspace=ws), n)
        hbm_row("silu_mul_quant (bf16 gate|up in, e4m3 codes out)", m, d_ff, t, m * d_ff * 5 + 4)
        del gu, q
        torch.cuda.empty_cache()
    for sub, (name, k, nn) in enumerate(synth.LLAMA3_8B_LINEARS):
        w = synth.weights_device(2, nn, k, sub=sub, row_multipliers=True)
        wq = torch.empty((nn, k), dtype=torch.uint8, device=dev)
        sw = torch.empty(nn, dtype=torch.float32, device=dev)
        t = timed(lambda: fp8.quant_dynamic_per_row(w, q=wq, scales=sw), 2)
        hbm_row("weight quantization per output channel (bf16 in, e4m3 codes and scales out)", nn, k, t,
                nn * k * 3 + 4 * nn, {"shape": name})
        del w, wq, sw
        torch.cuda.empty_cache()

    # e5m2 GEMMs: codes of the decode and prefill activations and the layer's weights in e5m2
    gemms = []
    for sub, (name, k, nn) in enumerate(synth.LLAMA3_8B_LINEARS):
        w = synth.weights_device(2, nn, k, sub=sub, row_multipliers=True)
        w_q, s_w = fp8.quant_weight(w, per_channel=True, fmt="e5m2")
        del w
        copies = [(w_q, s_w)] + [(w_q.clone(), s_w.clone()) for _ in range(ROTATE_DECODE - 1)]
        for m in (16, PREFILL_M):
            x = bf(synth.activations(2 if m == 16 else 3, m, k, sub=sub, outliers=True))
            a_q, s_a = fp8.quant_dynamic(x, fmt="e5m2")
            del x
            out = torch.empty((m, nn), dtype=torch.bfloat16, device=dev)
            use = copies if m == 16 else copies[:1]
            reps = 2 if m == 16 else 3

            def launch(use=use, a_q=a_q, s_a=s_a, out=out, reps=reps):
                for _ in range(reps):
                    for (wq_, sw_) in use:
                        fp8.scaled_mm(a_q, wq_, s_a, sw_, True, out=out, fmt_a="e5m2", fmt_w="e5m2")
            t = time_graph_per_launch(launch, reps * len(use), windows=5)
            r = {"M": m, "K": k, "N": nn, "shape": name, "us": round(t * 1e6, 2)}
            if m == 16:
                b = gemm_bytes(m, k, nn)
                r.update({"GBps": round(b / t / 1e9, 1), "frac_hbm": round(b / t / 1e9 / HBM_PEAK_GBS, 4)})
            else:
                tf = 2 * m * k * nn / t / 1e12
                r.update({"TFLOPs": round(tf, 1), "frac_fp8_peak": round(tf / FP8_PEAK_TFLOPS, 4),
                          "frac_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4)})
            gemms.append(r)
            del a_q, out
        del copies, w_q, s_w
        torch.cuda.empty_cache()
    dec = [g for g in gemms if g["M"] == 16]
    pre = [g for g in gemms if g["M"] != 16]
    dec_b = sum(gemm_bytes(16, g["K"], g["N"]) for g in dec)
    pre_f = sum(2 * g["M"] * g["K"] * g["N"] for g in pre)
    return {"workload": "the calls beyond the headline path at the Llama-3-8B layer's sizes (decode M=16, prefill "
                        "M=16384): producer-fused quantizations, static activation quantization, per-channel weight "
                        "quantization, e5m2 x e5m2 GEMMs (channelwise, exact sums); synthetic inputs",
            "quantizations": calls,
            "e5m2_gemms": gemms,
            "e5m2_decode_GBps": round(dec_b / (sum(g["us"] for g in dec) * 1e-6) / 1e9, 1),
            "e5m2_prefill_TFLOPs": round(pre_f / (sum(g["us"] for g in pre) * 1e-6) / 1e12, 1)}


def cpu_baseline(m, lin_shapes, row_frac=8, budget_s=8.0, threads=None):
    """Time the CPU oracle on a bounded sample of the same workload.

    Sample: each of the four linears restricted to its first N / row_frac
    output channels (same K, same M, same generators), quantized once
    (load-time work, untimed); then oracle steps (dynamic activation
    quantization + exact GEMM + epilogue for the four linears) repeat until
    about budget_s of timed work.  threads: the BLAS thread count (None:
    the library's default, all visible cores).  Returns (bytes, flops,
    seconds, threads, description) for the timed steps.
    """
    import oracle
    from threadpoolctl import threadpool_info, threadpool_limits
    prepared = []
    for sub, (name, k, n) in enumerate(lin_shapes):
        ns = max(1, n // row_frac)
        x = synth.activations(2, m, k, sub=sub, outliers=True)
        # the first ns rows of the full seeded weight (the streams are row-major)
        w = synth.weights(2, ns, k, sub=sub, row_multipliers=True)
        wq, sw = oracle.quant_weight(w, per_channel=True)
        prepared.append((name, k, ns, x, wq, sw))
    with threadpool_limits(limits=threads):
        used = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        done_bytes = done_flops = 0
        timed = 0.0
        steps = 0
        while steps == 0 or timed < budget_s:
            for (name, k, ns, x, wq, sw) in prepared:
                t0 = time.perf_counter()
                aq, sa = oracle.quant_dynamic(x)
                oracle.scaled_mm(aq, wq, sa, sw, True)
                timed += time.perf_counter() - t0
                done_bytes += quant_bytes(m, k) + gemm_bytes(m, k, ns)
                done_flops += 2 * m * k * ns
            steps += 1
    cpu = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), cpu)
    except OSError:
        pass
    desc = (f"{steps} oracle steps over the 4 linears at M={m} with N/{row_frac} output channels each "
            f"({timed:.1f} s timed; weight quantization untimed; element-wise NumPy on 1 thread, "
            f"fp64 BLAS matmul on {used} thread(s); {cpu}, {os.cpu_count()} logical CPUs visible)")
    return done_bytes, done_flops, timed, used, desc


def cpu_baselines(decode):
    """The oracle on all cores (the reported cpu_baseline) and on 1 thread."""
    shapes = synth.LLAMA3_8B_LINEARS
    cm = 16 if decode else 64          # prefill sample: 64 of the 16384 rows
    res = []
    for threads in (None, 1):
        nbytes, nflops, secs, used, desc = cpu_baseline(cm, shapes, threads=threads)
        if decode:
            cv, cu = nbytes / secs / 1e9, "GB/s"
        else:
            cv, cu = nflops / secs / 1e12, "TFLOP/s"
        res.append({"value": round(cv, 4), "unit": cu, "cores": used, "kind": "oracle", "sample": desc})
    all_cores, one = res
    all_cores["one_thread"] = one
    return all_cores


def run_chain(args):
    """The chained-linears workload: prefill of 16 prompts x 1024 tokens
    through the 32-layer stack, then decode steps at M = 16 whose input is the
    previous step's output (the first: each prompt's last position).  Decode
    steps replay one captured HIP graph; a few eager steps are timed too."""
    from fp8_w8a8_quantized_amd import chain
    steps = args.steps if args.steps is not None else 512
    warmup = args.warmup if args.warmup is not None else 2
    torch.cuda.set_device(0)
    log("building the 32-layer stack")
    c = chain.Chain(layers=32, accum=args.accum)
    prompts, seq = 16, 1024
    x = synth.bf16_bits_to_torch(synth.activations(5, prompts * seq, chain.D_MODEL, layer=100, outliers=True)).cuda()
    c.forward(x)                                            # allocate prefill buffers, warm up
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    h = c.forward(x)
    e1.record()
    torch.cuda.synchronize()
    prefill_ms = e0.elapsed_time(e1)
    start = h[seq - 1::seq].contiguous()
    xin, xout = start.clone(), torch.empty_like(start)
    for _ in range(warmup):
        c.forward(xin, out=xout)
    torch.cuda.synchronize()
    # eager decode steps (Python launches every kernel)
    n_eager = 8
    xin.copy_(start)
    e0.record()
    for _ in range(n_eager):
        c.forward(xin, out=xout)
        xin.copy_(xout)
    e1.record()
    torch.cuda.synchronize()
    eager_ms = e0.elapsed_time(e1) / n_eager
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        c.forward(xin, out=xout)
        xin.copy_(xout)
    xin.copy_(start)
    g.replay()
    torch.cuda.synchronize()
    xin.copy_(start)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    decode_ms = (time.perf_counter() - t0) * 1e3 / steps
    weight_bytes = 32 * sum(k * n for (_, k, n) in chain.SHAPES)
    prefill_flops = 32 * sum(2 * prompts * seq * k * n for (_, k, n) in chain.SHAPES)
    line = {
        "metric": METRIC + " -- chained-linears workload", "value": round(weight_bytes / (decode_ms * 1e-3) / 1e9, 2),
        "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": round(decode_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8e4m3 in, bf16 out; " + ("fp8 matrix-core sums (prefill)" if args.accum == "fp8"
                                            else "fp32-class sums (bf16 matrix cores on exact e4m3 values)"),
        "data": "synthetic",
        "config": {"workload": "32-layer Llama-3-8B-shaped stack of W8A8 linears (qkv, o, gate_up, down per layer, "
                               "channelwise weights, fresh dynamic activation scale before every linear; RMSNorm, "
                               "SiLU*mul and residual adds between them): 16 x 1024-token prefill, then decode "
                               "steps at M=16 fed by the previous step",
                   "layers": 32, "prefill_tokens": prompts * seq, "decode_M": prompts,
                   "launch": "decode: hip_graph per step; prefill: eager"},
        "chain": {"prefill_ms": round(prefill_ms, 2),
                  "prefill_tflops": round(prefill_flops / (prefill_ms * 1e-3) / 1e12, 1),
                  "decode_ms_per_step_graph": round(decode_ms, 4), "decode_ms_per_step_eager": round(eager_ms, 4),
                  "decode_total_s": round(decode_ms * steps / 1e3, 3),
                  "weight_bytes_per_decode_step": weight_bytes},
    }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", choices=["all", "decode", "prefill", "skinny", "mid_m", "chain", "next"],
                    default="all",
                    help="all (default): the decode line with prefill (both accumulation modes) and skinny "
                         "objects added; decode / prefill: that workload alone as the headline; skinny: the "
                         "small-M per-tensor GEMMs alone; mid_m: the GEMMs at M = 32 to 1024 alone; next: the "
                         "producer-fused, static and weight "
                         "quantizations and e5m2 GEMMs alone; chain: the 32-layer Llama-3-8B-shaped stack, "
                         "16 x 1024-token prefill, then decode steps at M=16 (--steps of them, default 512)")
    ap.add_argument("--accum", choices=["fp32", "fp8"], default="fp32",
                    help="GEMM accumulation of the decode / prefill / chain workloads: fp32-class sums (default) "
                         "or the fp8 matrix cores (M > 64)")
    ap.add_argument("--prefill-steps", type=int, default=5, help="timed prefill steps per mode in the default run")
    ap.add_argument("--eager", action="store_true",
                    help="launch every kernel from Python instead of replaying captured HIP graphs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after timing, run a fill, a device copy (3 times) and a sum over a buffer of this "
                         "many MiB, so that profiler byte counters can be scaled against kernels of known traffic")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the layer would shard column-parallel over N, each GPU holding a slice of the weight rows "
              "and their scales).", file=sys.stderr)
        sys.exit(2)
    if args.workload == "chain":
        return run_chain(args)
    torch.cuda.set_device(0)
    if args.workload == "next":
        line = {"metric": METRIC + " -- calls beyond the headline path", "unit": "GB/s", "n_gpus": 1,
                "higher_is_better": True, "data": "synthetic", "next": bench_next(args)}
        line["value"] = line["next"]["e5m2_decode_GBps"]
        print(json.dumps(line), flush=True)
        return
    if args.workload == "mid_m":
        line = {"metric": METRIC + " -- GEMMs between decode and prefill", "unit": "TFLOP/s", "n_gpus": 1,
                "higher_is_better": True, "data": "synthetic", "mid_m": bench_mid_m(args)}
        line["value"] = round(float(np.mean([r["TFLOPs"] for r in line["mid_m"]["gemms"]])), 1)
        print(json.dumps(line), flush=True)
        return
    if args.workload == "skinny":
        line = {"metric": METRIC + " -- small-M per-tensor GEMMs", "unit": "GB/s", "n_gpus": 1,
                "higher_is_better": True, "data": "synthetic", "skinny": bench_skinny(args)}
        if args.copy_calibration_mib > 0:
            copy_calibration(args.copy_calibration_mib)
        line["value"] = round(float(np.mean([r["GBps"] for r in line["skinny"]["gemms"] if r["M"] <= 16])), 1)
        print(json.dumps(line), flush=True)
        return
    decode = args.workload in ("all", "decode")
    m = 16 if decode else PREFILL_M
    steps = args.steps if args.steps is not None else (200 if decode else 20)
    warmup = args.warmup if args.warmup is not None else (20 if decode else 3)
    rotate = ROTATE_DECODE if decode else 1

    log(f"building inputs: {'decode' if decode else 'prefill'}, M={m}, rotate={rotate}")
    lin = build_layer(m, rotate, cfg=2 if decode else 3)
    ws = fp8.new_workspace()
    ms_per_step = time_steps(lin, ws, args.accum, steps, warmup, eager=args.eager)

    # Per-launch GEMM time: for each linear, a graph of back-to-back GEMM
    # launches over the weight copies, bracketed by HIP events on the stream
    # the launches run on; mean time per launch.
    reps = max(1, 16 // rotate) if decode else 3
    per_shape_s = gemm_times(lin, args.accum, reps)

    if args.copy_calibration_mib > 0:
        copy_calibration(args.copy_calibration_mib)

    step_bytes = sum(quant_bytes(m, L["k"]) + gemm_bytes(m, L["k"], L["n"]) for L in lin)
    step_flops = sum(2 * m * L["k"] * L["n"] for L in lin)
    per_launch_bytes = np.mean([gemm_bytes(m, L["k"], L["n"]) for L in lin])
    per_launch_flops = np.mean([2 * m * L["k"] * L["n"] for L in lin])
    avg_launch_s = float(np.mean(per_shape_s))
    per_shape_us = {L["name"]: round(per_shape_s[j] * 1e6, 2) for j, L in enumerate(lin)}

    if decode:
        value = step_bytes / (ms_per_step * 1e-3) / 1e9
        unit = "GB/s"
        achieved = per_launch_bytes / avg_launch_s / 1e9
        kernel = "gemm_skinny_kernel<4, 2, {false|true}, {false|true}, 0, 0> + gemm_skinny2_kernel<4, 1, true, 0, 0>"
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": recorded_traffic(kernel),
                "kernel": kernel, "avg_launch_us": round(avg_launch_s * 1e6, 2),
                "algorithmic_bytes_per_launch": int(per_launch_bytes), "per_shape_us": per_shape_us}
    else:
        value = step_flops / (ms_per_step * 1e-3) / 1e12
        unit = "TFLOP/s"
        achieved = per_launch_flops / avg_launch_s / 1e12
        kernel = f"gemm_mfma_kernel<4, {'false' if args.accum == 'fp8' else 'true'}, true, 0, 0>"
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / FP8_PEAK_TFLOPS, 4), "traffic": recorded_traffic(kernel),
                "kernel": kernel, "avg_launch_us": round(avg_launch_s * 1e6, 2),
                "algorithmic_flops_per_launch": int(per_launch_flops), "per_shape_us": per_shape_us}

    line = {
        "metric": METRIC, "value": round(value, 2), "unit": unit, "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8e4m3 in, bf16 out; " + ("fp8 matrix-core sums" if args.accum == "fp8" and not decode
                                              else "fp32-class sums (bf16 matrix cores on exact e4m3 values)"),
        "data": "synthetic",
        "config": {"workload": f"llama3-8b {'decode' if decode else 'prefill'} linears (qkv, o, gate_up, down), "
                               f"M={m}, channelwise weight scales, dynamic per-tensor activation scale"
                               + (f", weights rotated over {rotate} layer copies" if rotate > 1 else ""),
                   "M": m, "shapes_kn": [[L["k"], L["n"]] for L in lin],
                   "launch": "eager" if args.eager else "hip_graph"},
        "roofline": roof,
    }
    if args.workload == "all":
        line["prefill"] = bench_prefill_modes(lin, args)
        del lin
        torch.cuda.empty_cache()
        line["skinny"] = bench_skinny(args)
        line["mid_m"] = bench_mid_m(args)
        line["next"] = bench_next(args)
    else:
        del lin
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baselines(decode)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
