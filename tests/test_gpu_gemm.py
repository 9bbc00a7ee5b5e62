"""Scaled GEMM on the GPU vs the exact CPU oracle (element-wise tolerance)."""
import numpy as np
import pytest
import torch

import oracle
import fp8_w8a8_quantized_amd as fp8
from fp8_w8a8_quantized_amd import synth
from _helpers import say, dev_bf16, host_u8, host_f32, host_bf16_bits, assert_gemm_close

pytestmark = pytest.mark.gpu


def _prepare(cfg, m, k, n, per_channel, outliers=False, rowmul=False, with_bias=False, sub=0):
    """Inputs from the seeded generators, quantized independently on each side;
    the GPU's quantized operands must equal the oracle's byte for byte."""
    x = synth.activations(cfg, m, k, sub=sub, outliers=outliers)
    w = synth.weights(cfg, n, k, sub=sub, row_multipliers=rowmul)
    b = synth.bias(cfg, n, sub=sub) if with_bias else None
    a_q, s_a = fp8.quant_dynamic(dev_bf16(x))
    w_q, s_w = fp8.quant_weight(dev_bf16(w), per_channel)
    aq_ref, sa_ref = oracle.quant_dynamic(x)
    wq_ref, sw_ref = oracle.quant_weight(w, per_channel)
    torch.cuda.synchronize()
    assert host_f32(s_a)[0] == sa_ref and np.array_equal(host_u8(a_q), aq_ref)
    assert np.array_equal(host_f32(s_w), sw_ref) and np.array_equal(host_u8(w_q), wq_ref)
    bias_d = dev_bf16(b) if b is not None else None
    return dict(a_q=a_q, s_a=s_a, w_q=w_q, s_w=s_w, bias=bias_d, bias_bits=b,
                aq=aq_ref, sa=sa_ref, wq=wq_ref, sw=sw_ref)


def _run_and_check(d, per_channel, rows=None, accum="fp32"):
    out = fp8.scaled_mm(d["a_q"], d["w_q"], d["s_a"], d["s_w"], per_channel, d["bias"], accum=accum)
    torch.cuda.synchronize()
    ob = host_bf16_bits(out)
    aq = d["aq"] if rows is None else d["aq"][rows]
    ref = oracle.scaled_mm(aq, d["wq"], d["sa"], d["sw"], per_channel, d["bias_bits"])
    return assert_gemm_close(ob, ref, d["aq"], d["sa"], d["wq"], d["sw"], per_channel, rows=rows,
                             bias_bits=d["bias_bits"], accum=accum), out


# ------------------------------------------------------------- skinny (M <= 64)
@pytest.mark.parametrize("m", [1, 3, 7, 13, 16])
@pytest.mark.parametrize("k,n", [(4096, 4100), (4096, 1030), (4096, 4096)])
def test_skinny_per_tensor_unaligned(m, k, n):
    say("skinny per-tensor", m, k, n)
    d = _prepare(4, m, k, n, per_channel=False)
    _run_and_check(d, False)


@pytest.mark.parametrize("m,k,n", [(16, 4096, 6144), (16, 14336, 4096), (5, 4096, 28672)])
def test_skinny_per_channel_llama_shapes(m, k, n):
    say("skinny per-channel", m, k, n)
    d = _prepare(2, m, k, n, per_channel=True, outliers=True, rowmul=True, with_bias=(m == 5))
    _run_and_check(d, True)


@pytest.mark.parametrize("m,k,n,pc", [(16, 4096, 16400, True), (3, 2048, 16392, False), (13, 1024, 16400, True),
                                      (16, 4096, 28672, False), (9, 4096, 20000, True), (16, 1024, 30000, False),
                                      (11, 4096, 14305, True), (16, 4096, 14304, False)])
def test_skinny_large_n_ragged(m, k, n, pc):
    """N from the two-block threshold up (N >= 14305 on 256 CUs) with K below
    8192: two weight blocks per wave, 24, 28 or 32 rows per workgroup, a last
    workgroup partly past N (14305: 511 workgroups of 28 rows, the last with
    25), plain and non-temporal weight loads, per-tensor and channelwise;
    N = 14304, one below the threshold, takes the one-block kernel."""
    say("skinny large n", m, k, n, pc)
    d = _prepare(6, m, k, n, per_channel=pc, rowmul=pc, with_bias=pc)
    _run_and_check(d, pc)


@pytest.mark.parametrize("m,k,n", [(7, 8192, 1030), (3, 8208, 257), (16, 16384, 100)])
def test_skinny_long_k_interleaved(m, k, n):
    """K >= 8192 with weights under 32 MiB: K steps interleaved across the
    waves, plain loads; ragged N and M, and a K whose last step is partial
    (8208 = 32 steps of 256 + 16)."""
    say("skinny long K", m, k, n)
    d = _prepare(6, m, k, n, per_channel=True, outliers=True, rowmul=True, with_bias=(m == 3))
    _run_and_check(d, True)


@pytest.mark.parametrize("m,k,n", [(1, 1, 1), (2, 7, 3), (16, 100, 17), (9, 272, 33), (16, 16, 16), (4, 4099, 40)])
def test_skinny_tiny_and_ragged_k(m, k, n):
    say("skinny ragged", m, k, n)
    d = _prepare(4, m, k, n, per_channel=True, with_bias=True, rowmul=True)
    _run_and_check(d, True)


# -------------------------------------------------- mid M (skinny over M blocks)
@pytest.mark.parametrize("m,k,n", [(17, 4096, 1030), (33, 512, 4100), (64, 1024, 300),
                                   (40, 14336, 2401), (20, 4096, 8200), (48, 1040, 777), (63, 8208, 513),
                                   (57, 4096, 16)])
def test_mid_m(m, k, n):
    """16 < M <= 64 on the multi-block skinny kernel: two, three or four
    16-row blocks of M per workgroup in one grid row, or two grid rows of 2
    blocks where one row would have few workgroups (N <= 2048 here); shapes
    with at least 32 MiB of weights (non-temporal loads), interleaved and
    contiguous K steps, K tails that are not whole 256-byte steps, a ragged
    N and a partial last block of M."""
    say("mid m", m, k, n)
    d = _prepare(4, m, k, n, per_channel=False, with_bias=True)
    _run_and_check(d, False)


@pytest.mark.parametrize("m,k,n", [(65, 1024, 4100), (81, 2048, 3000), (129, 1024, 4104), (190, 512, 2056),
                                   (64, 2048, 6144), (50, 1024, 1030), (33, 512, 2040)])
def test_skinny_grid_rows_share_the_blocks(m, k, n):
    """Past 64 rows the multi-block kernel runs ceil(M / 64) grid rows and
    spreads the 16-row blocks of M evenly over them: 65 and 81 rows as two
    grid rows of 3 blocks (the second with 1 and 33 rows), 129 as three of 3,
    190 as three of 4.  From 33 to 64 rows, on a 256-CU part, two grid rows
    replace one where a single row has few workgroups: 64 x 6144 as two rows
    of 2 blocks, 50 x 1030 as two of 2 (the second with 18 rows), 33 x 2040
    (128 workgroups per row) as two of 2 (the second with 1 row).  The grid
    rows of one weight block are dealt to one XCD.  Per-channel scales, a
    bias, ragged N."""
    say("skinny grid rows", m, k, n)
    d = _prepare(10, m, k, n, per_channel=True, rowmul=True, with_bias=True, sub=m)
    _run_and_check(d, True)


# ------------------------------------- wide skinny kernel (16 < M <= 64, wide N)
@pytest.mark.parametrize("m,k,n,pc,bias", [
    (33, 4096, 14336, True, True),    # M > 32, N = 56 x CUs: one row in the third block of M
    (40, 1024, 14400, False, False),  # plain weight loads (under 32 MiB), per-tensor
    (64, 2048, 14344, True, True),    # the last workgroup: wave 0 holds 8 rows, waves 1-3 start past N
    (17, 4096, 28672, True, False),   # M > 16, N = 112 x CUs: one row in the second block
    (24, 1040, 28680, False, True),   # a ragged k step (K = 4 x 256 + 16)
    (48, 4096, 28676, True, True),    # N % 8 == 4: 8-byte stores, the last columns element by element
    (63, 4096, 14339, True, True),    # odd N: every row of the last block element by element
    (40, 16, 14400, True, True),      # one partial k step (K = 16): the pipeline's second slot never loads
    (50, 272, 28672, True, True),     # one step and a 16-byte tail; 48 < M <= 64 below N = 57344
])
def test_wide_skinny_kernel(m, k, n, pc, bias):
    """The wide skinny kernel (each wave its own 16-row weight block over all
    of K, the activation steps shared through LDS; on a 256-CU part it runs
    for M > 32 with N >= 14336 and for M > 16 with N >= 28672): ragged M, N
    and K, per-tensor and per-channel scales, with and without bias."""
    say("wide skinny", m, k, n, pc, bias)
    d = _prepare(9, m, k, n, per_channel=pc, outliers=pc, rowmul=pc, with_bias=bias)
    _run_and_check(d, pc)


@pytest.mark.parametrize("m,n", [(32, 14336), (33, 14336), (33, 14335), (16, 28672), (17, 28672), (17, 28671)])
def test_wide_skinny_kernel_bounds(m, n):
    """Both sides of the wide kernel's bounds (on a 256-CU part): 33 x 14336
    and 17 x 28672 run it; M = 32 and N = 14335 stay on the multi-block
    kernel, M = 16 on the two-block kernel, N = 28671 with M = 17 on the
    multi-block kernel.  Pitched operands and output (the kernels index rows
    by pitch, not by K or N)."""
    k = 1024
    say("wide bounds", m, k, n)
    d = _prepare(9, m, k, n, per_channel=True, rowmul=True, with_bias=True, sub=m)
    a = torch.zeros((m, k + 48), dtype=torch.uint8, device="cuda")
    a[:, :k] = d["a_q"]
    w = torch.zeros((n, k + 32), dtype=torch.uint8, device="cuda")
    w[:, :k] = d["w_q"]
    out = torch.zeros((m, n + 24), dtype=torch.bfloat16, device="cuda")[:, :n]
    fp8.scaled_mm(a[:, :k], w[:, :k], d["s_a"], d["s_w"], True, d["bias"], out=out)
    torch.cuda.synchronize()
    ref = oracle.scaled_mm(d["aq"], d["wq"], d["sa"], d["sw"], True, d["bias_bits"])
    assert_gemm_close(host_bf16_bits(out), ref, d["aq"], d["sa"], d["wq"], d["sw"], True, bias_bits=d["bias_bits"])


# ------------------------------ matrix-core GEMM (M > 64 with enough output tiles)
@pytest.mark.parametrize("accum", ["fp32", "fp8"])
@pytest.mark.parametrize("m,k,n,pc", [
    (256, 256, 12288, False), (512, 4096, 1024, True), (300, 4096, 4100, False),
    (777, 1040, 520, True), (65, 128, 24576, False), (1000, 4096, 6144, True), (2048, 1024, 8192, True)])
def test_mfma_gemm(m, k, n, pc, accum):
    """The matrix-core GEMM: M > 256, or M of 65 and 256 with N large enough
    that the call does not give the problem to the skinny kernel (one row of
    tiles, mostly past M for M = 65).  All but 2048 x 1024 -> 8192 (256 tiles
    of 256 x 256) run 128 x 128 tiles, too few 256 x 256 ones; 1000 x 4096 ->
    6144 runs 384 of them, two workgroups per CU."""
    say("mfma", m, k, n, pc, accum)
    d = _prepare(3, m, k, n, per_channel=pc, outliers=pc, rowmul=pc, with_bias=(m % 2 == 0))
    _run_and_check(d, pc, accum=accum)


@pytest.mark.parametrize("accum", ["fp32", "fp8"])
@pytest.mark.parametrize("m,k,n", [(65, 4096, 1030), (128, 4096, 4096), (256, 256, 256), (200, 14336, 300),
                                   (96, 4096, 8192), (96, 4096, 14336), (256, 4096, 6144), (320, 4096, 4096),
                                   (1024, 1024, 4100), (64, 4096, 28672), (48, 4096, 28672), (57, 1024, 24576),
                                   (56, 1024, 57344), (49, 512, 57352), (96, 1024, 10240), (128, 1024, 10240)])
def test_mid_m_problems_on_each_kernel(m, k, n, accum):
    """Around the skinny kernels' bounds: problems too small for the
    matrix-core tiles (64 < M <= 256 and N x the skinny kernel's 16-row block
    slots below 81920: 96 x 10240 has 2 grid rows of 3, 128 x 10240 of 4)
    run on the skinny kernel in grid rows of up to 64 rows of M, as do
    M <= 64 but for 48 < M <= 64 with N >= 57344 (two rounds of 128 x 128
    tiles and more);
    the skinny kernels sum with fp32-class precision whatever the mode asked
    for (both modes meet the fp32 bound and give the same bits).  The others
    run on the matrix-core GEMM with 128 x 128 tiles (too few 256 x 256 ones
    to occupy the GPU): M = 96 and 256 on N = 14336 and 6144, M = 320 and
    1024 with ragged N, M = 56 and 49 on N of 57344 and more.  M = 48 to 64
    on N of 24576 and 28672 run the wide skinny kernel."""
    say("mid m", m, k, n, accum)
    d = _prepare(7, m, k, n, per_channel=True, outliers=True, rowmul=True, with_bias=True)
    blocks = (m + 15) // 16
    rows = (blocks + 3) // 4
    slots = rows * ((blocks + rows - 1) // rows)  # grid rows x blocks per grid row of the skinny kernel
    skinny = (m <= 64 and not (m > 48 and n >= 57344)) or (64 < m <= 256 and n * slots < 81920)
    out = fp8.scaled_mm(d["a_q"], d["w_q"], d["s_a"], d["s_w"], True, d["bias"], accum=accum)
    torch.cuda.synchronize()
    ref = oracle.scaled_mm(d["aq"], d["wq"], d["sa"], d["sw"], True, d["bias_bits"])
    assert_gemm_close(host_bf16_bits(out), ref, d["aq"], d["sa"], d["wq"], d["sw"], True, bias_bits=d["bias_bits"],
                      accum="fp32" if skinny else accum)
    if skinny and accum == "fp8":
        exact = fp8.scaled_mm(d["a_q"], d["w_q"], d["s_a"], d["s_w"], True, d["bias"], accum="fp32")
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), exact.view(torch.int16))


@pytest.mark.parametrize("accum", ["fp32", "fp8"])
@pytest.mark.parametrize("k,n", [(128, 4104), (256, 4101), (400, 4104)])
def test_mfma_gemm_several_tiles_per_workgroup_short_k(k, n, accum):
    """17 x 17 tiles (more than one per workgroup on a 256-CU part) with one,
    two and four (ragged) k steps per tile, vector and scalar output stores:
    the wait counts at tile changes (stores still in flight, the fp8 mode's
    prefetch loads) and the next tile's first step loaded during the last."""
    m = 4352
    say("mfma several tiles", m, k, n, accum)
    d = _prepare(5, m, k, n, per_channel=True, rowmul=True, with_bias=True)
    rows = np.r_[0:m:7, m - 9:m]
    _run_and_check(d, True, rows=rows, accum=accum)


@pytest.mark.parametrize("accum", ["fp32", "fp8"])
def test_mfma_gemm_k_not_multiple_of_128(accum):
    d = _prepare(3, 320, 4096 + 48, 512, per_channel=True, rowmul=True)
    _run_and_check(d, True, accum=accum)


def test_m_above_64_with_a_weight_pitch_the_matrix_core_kernel_refuses():
    """M = 80 with W rows 2^23 + 16 bytes apart: a 256-row weight panel would
    span 2 GiB, past the matrix-core kernel's 32-bit buffer offsets, so the
    multi-block skinny kernel runs M in two grid rows of 3 blocks of 16 rows
    (the second one partly past M).  Only the first K bytes of each weight
    row are codes."""
    m, k, n, ldw = 80, 4096, 24, (1 << 23) + 16
    say("pitched weight, M > 64", m, k, n, ldw)
    d = _prepare(9, m, k, n, per_channel=True, outliers=True, rowmul=True, with_bias=True)
    buf = torch.zeros((n, ldw), dtype=torch.uint8, device="cuda")
    buf[:, :k].copy_(d["w_q"])
    d["w_q"] = buf[:, :k]
    assert d["w_q"].stride(0) == ldw
    _run_and_check(d, True)
    del buf


@pytest.mark.timeout(600)
def test_m_over_one_skinny_grid_slice():
    """M = 1,048,580 rows with K = 24 (not a multiple of 16, so the
    byte-granular skinny kernel): the rows go out in slices of 65535 blocks
    of 16 (the grid's second dimension), here two, the second of 20 rows."""
    m, k, n = 65535 * 16 + 20, 24, 40
    say("two skinny slices", m, k, n)
    d = _prepare(10, m, k, n, per_channel=True, rowmul=True, with_bias=True)
    _run_and_check(d, True)


@pytest.mark.timeout(600)
def test_activation_codes_past_4_gib_sampled_rows():
    """A = 262,221 x 16,384 codes (4.3 GB): the matrix-core kernel's tiles
    start past 2 and 4 GiB of A, so their base addresses need 64 bits.  The
    bf16 activation is drawn on the device (N(0,1), -80 planted last, so the
    scale is fl32(80/448)); the oracle quantizes the sampled rows itself from
    their bf16 values, and the GPU's codes of those rows must equal its own.
    The GEMM is checked on rows around the 2 and 4 GiB marks, the first and
    the last (ragged) tile, in both accumulation modes."""
    m, k, n = 262144 + 77, 16384, 264
    gen = torch.Generator(device="cuda")
    gen.manual_seed(13)
    x = torch.randn((m, k), generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    x[-1, -1] = -80.0
    torch.cuda.synchronize()
    marks = [(1 << 31) // k, (1 << 32) // k]
    rows = np.array(sorted({0, 1, 255, 256, m - 78, m - 77, m - 2, m - 1,
                            *[r + d for r in marks for d in (-1, 0, 1)]}))
    say("A past 4 GiB", m, k, n, "sampled rows", rows.tolist())
    xs = host_bf16_bits(x[torch.from_numpy(rows).cuda()])
    s_ref = oracle.scale_from_amax(np.float32(80.0))
    aq_rows = oracle.quant_static(xs, s_ref)
    a_q, s_a = fp8.quant_dynamic(x)
    del x
    w = synth.weights(11, n, k, row_multipliers=True)
    b = synth.bias(11, n)
    w_q, s_w = fp8.quant_weight(dev_bf16(w), True)
    wq_ref, sw_ref = oracle.quant_weight(w, True)
    torch.cuda.synchronize()
    assert host_f32(s_a)[0] == s_ref
    assert np.array_equal(host_u8(a_q[torch.from_numpy(rows).cuda()]), aq_rows)
    assert np.array_equal(host_f32(s_w), sw_ref) and np.array_equal(host_u8(w_q), wq_ref)
    ref = oracle.scaled_mm(aq_rows, wq_ref, s_ref, sw_ref, True, b)
    for accum in ("fp32", "fp8"):
        say("  accumulation", accum)
        out = fp8.scaled_mm(a_q, w_q, s_a, s_w, True, dev_bf16(b), accum=accum)
        torch.cuda.synchronize()
        ob = host_bf16_bits(out[torch.from_numpy(rows).cuda()])
        del out
        assert_gemm_close(ob, ref, aq_rows, s_ref, wq_ref, sw_ref, True, bias_bits=b, accum=accum)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("m,k,n", [(16, 16384, 270000), (16, 7936, 560000), (300, 16384, 270000)])
def test_weights_past_4_gib_sampled_columns(m, k, n):
    """W of 4.4 GB: the skinny kernel with interleaved K steps (K = 16384),
    the two-block skinny kernel (K = 7936, under 32 steps of 256) and the
    matrix-core kernel (M = 300) address weight rows past 2 and 4 GiB.  The
    bf16 weights are drawn on the device (N(0, 0.02)); channelwise scales
    depend on their own row only, so the oracle quantizes the sampled weight
    rows itself (codes and scales must equal the GPU's) and checks the
    output columns of those rows."""
    gen = torch.Generator(device="cuda")
    gen.manual_seed(14)
    w = torch.randn((n, k), generator=gen, device="cuda", dtype=torch.bfloat16) * 0.02
    torch.cuda.synchronize()
    marks = [(1 << 31) // k, (1 << 32) // k]
    cols = np.array(sorted({0, 1, n - 17, n - 2, n - 1, *[r + d for r in marks for d in (-1, 0, 1)]}))
    say("W past 4 GiB", m, k, n, "sampled rows", cols.tolist())
    idx = torch.from_numpy(cols).cuda()
    w_rows = host_bf16_bits(w[idx])
    w_q, s_w = fp8.quant_weight(w, True)
    del w
    wq_ref, sw_ref = oracle.quant_weight(w_rows, True)
    x = synth.activations(12, m, k, outliers=True)
    a_q, s_a = fp8.quant_dynamic(dev_bf16(x))
    aq_ref, sa_ref = oracle.quant_dynamic(x)
    torch.cuda.synchronize()
    assert np.array_equal(host_f32(s_w[idx]), sw_ref) and np.array_equal(host_u8(w_q[idx]), wq_ref)
    assert host_f32(s_a)[0] == sa_ref and np.array_equal(host_u8(a_q), aq_ref)
    ref = oracle.scaled_mm(aq_ref, wq_ref, sa_ref, sw_ref, True)
    for accum in (("fp32", "fp8") if m > 64 else ("fp32",)):
        say("  accumulation", accum)
        out = fp8.scaled_mm(a_q, w_q, s_a, s_w, True, accum=accum)
        torch.cuda.synchronize()
        ob = host_bf16_bits(out[:, idx])
        del out
        assert_gemm_close(ob, ref, aq_ref, sa_ref, wq_ref, sw_ref, True, accum=accum)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("k", [64, 24])
def test_output_past_4_gib_sampled_rows(k):
    """out = 65,549 x 32,776 bf16 (4.3 GB): the matrix-core kernel's tile
    stores (K = 64) and the byte-granular skinny kernel's row stores (K = 24)
    land past 2 and 4 GiB of the output.  Inputs come from the seeded
    generators and are quantized on both sides (codes compared in full);
    output rows around the 2 and 4 GiB marks, the first and the last rows
    are checked."""
    m, n = 65536 + 13, 32776
    row_bytes = n * 2
    marks = [(1 << 31) // row_bytes, (1 << 32) // row_bytes]
    rows = np.array(sorted({0, 1, m - 14, m - 2, m - 1, *[r + d for r in marks for d in (-1, 0, 1)]}))
    say("output past 4 GiB", m, k, n, "sampled rows", rows.tolist())
    d = _prepare(13, m, k, n, per_channel=True, rowmul=True, with_bias=True)
    out = fp8.scaled_mm(d["a_q"], d["w_q"], d["s_a"], d["s_w"], True, d["bias"])
    torch.cuda.synchronize()
    ob = host_bf16_bits(out[torch.from_numpy(rows).cuda()])
    del out
    ref = oracle.scaled_mm(d["aq"][rows], d["wq"], d["sa"], d["sw"], True, d["bias_bits"])
    assert_gemm_close(ob, ref, d["aq"][rows], d["sa"], d["wq"], d["sw"], True, bias_bits=d["bias_bits"])


def _device_codes(gen, shape):
    """Uniformly random finite e4m3 codes drawn on the device (the NaN codes
    0x7F and 0xFF become 0), filled 1 GiB at a time."""
    t = torch.empty(shape, dtype=torch.uint8, device="cuda")
    flat = t.view(-1)
    for i in range(0, flat.numel(), 1 << 30):
        sl = flat[i:i + (1 << 30)]
        sl.random_(0, 256, generator=gen)
        sl.masked_fill_((sl & 0x7F) == 0x7F, 0)
    return t


@pytest.mark.timeout(600)
def test_rows_up_to_2_pow_31_on_the_matrix_core_kernel():
    """M = 2^31 - 1, the most rows the call takes (K = 16, N = 8: 32 GiB of
    activation codes and a 32 GiB output).  Counting the tiles adds up to a
    tile's rows to M, past 2^31, so it has to run in 64 bits.  fp32-class sums
    run 128 x 128 tiles here and fp8 sums 256 x 256 ones, so both tile sizes
    are covered.  Rows at the start, around 2^30 and in the last (ragged)
    tiles are checked against the oracle."""
    m, k, n = (1 << 31) - 1, 16, 8
    gen = torch.Generator(device="cuda")
    gen.manual_seed(21)
    a_q = _device_codes(gen, (m, k))
    torch.cuda.synchronize()
    rows = np.array(sorted({0, 1, 127, 128, 255, 256, (1 << 30) - 1, 1 << 30, m - 257, m - 256, m - 255,
                            m - 128, m - 127, m - 2, m - 1}))
    say("M = 2^31 - 1", m, k, n, "sampled rows", rows.tolist())
    idx = torch.from_numpy(rows).cuda()
    aq_rows = host_u8(a_q[idx])
    w = synth.weights(11, n, k, row_multipliers=True)
    b = synth.bias(11, n)
    w_q, s_w = fp8.quant_weight(dev_bf16(w), True)
    wq_ref, sw_ref = oracle.quant_weight(w, True)
    s_a = torch.tensor([0.0625], dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    assert np.array_equal(host_f32(s_w), sw_ref) and np.array_equal(host_u8(w_q), wq_ref)
    ref = oracle.scaled_mm(aq_rows, wq_ref, np.float32(0.0625), sw_ref, True, b)
    for accum in ("fp32", "fp8"):
        say("  accumulation", accum)
        out = fp8.scaled_mm(a_q, w_q, s_a, s_w, True, dev_bf16(b), accum=accum)
        torch.cuda.synchronize()
        ob = host_bf16_bits(out[idx])
        del out
        assert_gemm_close(ob, ref, aq_rows, np.float32(0.0625), wq_ref, sw_ref, True, bias_bits=b, accum=accum)


@pytest.mark.timeout(600)
def test_columns_up_to_2_pow_31_on_the_skinny_kernel():
    """N = 2^31 - 1, the most output columns the call takes (M = 2, K = 2:
    the byte-granular skinny kernel; 4 GiB of weight codes, per-channel
    scales (8 GiB), a bias (4 GiB) and an 8 GiB output).  The call runs in
    column slices of 2^25, since one launch's threads must stay below 2^32,
    and counts its column blocks in 64 bits.  Columns at the start, at slice
    boundaries, around 2^30 and in the last (ragged) block are checked
    against the oracle."""
    m, k, n = 2, 2, (1 << 31) - 1
    gen = torch.Generator(device="cuda")
    gen.manual_seed(22)
    w_q = _device_codes(gen, (n, k))
    s_w = torch.empty(n, dtype=torch.float32, device="cuda").uniform_(0.25, 4.0, generator=gen)
    bias = torch.empty(n, dtype=torch.bfloat16, device="cuda").normal_(generator=gen)
    torch.cuda.synchronize()
    cols = np.array(sorted({0, 1, 15, 16, (1 << 25) - 1, 1 << 25, (1 << 25) + 1, (1 << 30) - 1, 1 << 30,
                            n - 17, n - 16, n - 15, n - 2, n - 1}))
    say("N = 2^31 - 1", m, k, n, "sampled columns", cols.tolist())
    idx = torch.from_numpy(cols).cuda()
    wq_cols = host_u8(w_q[idx])
    sw_cols = host_f32(s_w[idx])
    b_cols = host_bf16_bits(bias[idx])
    codes = np.arange(256, dtype=np.uint8)
    codes = codes[(codes & 0x7F) != 0x7F]
    aq = np.random.default_rng(22).choice(codes, size=(m, k)).astype(np.uint8)
    s_a = torch.tensor([0.5], dtype=torch.float32, device="cuda")
    out = fp8.scaled_mm(torch.from_numpy(aq).cuda(), w_q, s_a, s_w, True, bias)
    torch.cuda.synchronize()
    ob = host_bf16_bits(out[:, idx])
    del out
    ref = oracle.scaled_mm(aq, wq_cols, np.float32(0.5), sw_cols, True, b_cols)
    assert_gemm_close(ob, ref, aq, np.float32(0.5), wq_cols, sw_cols, True, bias_bits=b_cols)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("m,n", [(13, 130), (40, 72), (300, 520)])
def test_longest_k_the_oracle_sums_exactly(m, n):
    """K = 131072, near the oracle's exactness limit (K < 171,196).  It
    exercises the skinny kernel's longest interleaved K loop (M = 13, one
    block of M; M = 40, three blocks per weight step), the matrix-core
    kernel with 1,024 k steps per tile in both accumulation modes, and the
    two-launch quantizer over up to 39 M elements.  The float32 sums round
    once per matrix-core product (32 or 64 k at a time), a few thousand
    times per output, far inside the tolerance."""
    k = 131072
    say("longest K", m, k, n)
    d = _prepare(8, m, k, n, per_channel=True, outliers=True, rowmul=True, with_bias=True)
    for accum in (("fp32", "fp8") if m > 64 else ("fp32",)):
        say("  accumulation", accum)
        _run_and_check(d, True, accum=accum)


@pytest.mark.parametrize("m", [16, 300])
@pytest.mark.parametrize("accum", ["fp32", "fp8"])
def test_every_code_through_identity_weight(m, accum):
    """W_q = 0x38 * I (weight 1.0) makes each output one product:
    out[m, n] = dec(A_q[m, n]) * s_a * s_w exactly, for all 254 finite codes."""
    k = 256
    codes = np.arange(256, dtype=np.uint8)
    codes[[0x7F, 0xFF]] = 0
    rng = np.random.default_rng(m)
    a = np.stack([rng.permutation(codes) for _ in range(m)])
    w = np.where(np.eye(k, dtype=bool), np.uint8(0x38), np.uint8(0))
    s_a = torch.tensor([0.25], dtype=torch.float32, device="cuda")
    s_w = torch.tensor([2.0], dtype=torch.float32, device="cuda")
    out = fp8.scaled_mm(torch.from_numpy(a).cuda(), torch.from_numpy(w).cuda(), s_a, s_w, False, accum=accum)
    torch.cuda.synchronize()
    want = oracle.decode(a) * 0.5
    got = oracle.bf16_bits_to_f32(host_bf16_bits(out)).astype(np.float64)
    assert np.array_equal(got, want)


def test_unaligned_layout_falls_back_correctly():
    """Row pitches that are not multiples of 16 bytes (M > 64): generic path."""
    m, k, n = 130, 1000, 200
    x = synth.activations(8, m, k); w = synth.weights(8, n, k)
    xa = torch.zeros((m, 1003), dtype=torch.bfloat16, device="cuda"); xa[:, :k] = dev_bf16(x)
    wa = torch.zeros((n, 1001), dtype=torch.bfloat16, device="cuda"); wa[:, :k] = dev_bf16(w)
    a_q, s_a = fp8.quant_dynamic(xa[:, :k], q=torch.empty((m, 1001), dtype=torch.uint8, device="cuda")[:, :k])
    w_q, s_w = fp8.quant_dynamic(wa[:, :k], q=torch.empty((n, 1005), dtype=torch.uint8, device="cuda")[:, 1:k + 1])
    outbuf = torch.full((m, n + 7), -7.0, dtype=torch.bfloat16, device="cuda")
    out = fp8.scaled_mm(a_q, w_q, s_a, s_w, False, out=outbuf[:, 3:n + 3])
    torch.cuda.synchronize()
    aq, sa = oracle.quant_dynamic(x); wq, sw = oracle.quant_weight(w, False)
    ref = oracle.scaled_mm(aq, wq, sa, sw, False)
    assert_gemm_close(host_bf16_bits(out), ref, aq, sa, wq, sw, False)
    ob = outbuf.float().cpu().numpy()
    assert np.all(ob[:, :3] == -7.0) and np.all(ob[:, n + 3:] == -7.0)


@pytest.mark.parametrize("accum", ["fp32", "fp8"])
def test_mfma_padded_pitches_and_output_view(accum):
    """Matrix-core path with row pitches larger than K and N (16-byte
    multiples), a k tail, several tiles, and an output sub-view whose guard
    columns must stay untouched."""
    m, k, n = 600, 1040, 520
    x = synth.activations(9, m, k, outliers=True); w = synth.weights(9, n, k, row_multipliers=True)
    b = synth.bias(9, n)
    a_q, s_a = fp8.quant_dynamic(dev_bf16(x), q=torch.empty((m, 1072), dtype=torch.uint8, device="cuda")[:, :k])
    w_q, s_w = fp8.quant_dynamic_per_row(dev_bf16(w), q=torch.empty((n, 1056), dtype=torch.uint8, device="cuda")[:, :k])
    outbuf = torch.full((m, 536 + 16), -7.0, dtype=torch.bfloat16, device="cuda")
    out = fp8.scaled_mm(a_q, w_q, s_a, s_w, True, dev_bf16(b), out=outbuf[:, 8:8 + n], accum=accum)
    torch.cuda.synchronize()
    aq, sa = oracle.quant_dynamic(x); wq, sw = oracle.quant_weight(w, True)
    assert np.array_equal(host_u8(a_q), aq) and np.array_equal(host_u8(w_q), wq)
    ref = oracle.scaled_mm(aq, wq, sa, sw, True, b)
    assert_gemm_close(host_bf16_bits(out), ref, aq, sa, wq, sw, True, bias_bits=b, accum=accum)
    ob = outbuf.float().cpu().numpy()
    assert np.all(ob[:, :8] == -7.0) and np.all(ob[:, 8 + n:] == -7.0)


# -------------------------------------------------------------- invariants
@pytest.mark.parametrize("m,n", [(16, 4096), (512, 1024)])
def test_per_channel_equal_scales_bit_exact_with_per_tensor(m, n):
    k = 4096
    d = _prepare(1, m, k, n, per_channel=False)
    sig = d["s_w"]
    s_vec = sig.repeat(n).contiguous()
    o1 = fp8.scaled_mm(d["a_q"], d["w_q"], d["s_a"], sig, False)
    o2 = fp8.scaled_mm(d["a_q"], d["w_q"], d["s_a"], s_vec, True)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_output_canaries_and_pitch():
    m, k, n = 300, 512, 1030
    d = _prepare(5, m, k, n, per_channel=True, rowmul=True)
    buf = torch.full((m + 2, n + 9), 3.0, dtype=torch.bfloat16, device="cuda")
    out = buf[1:m + 1, 4:n + 4]
    fp8.scaled_mm(d["a_q"], d["w_q"], d["s_a"], d["s_w"], True, out=out)
    torch.cuda.synchronize()
    h = buf.float().cpu().numpy()
    assert np.all(h[0] == 3.0) and np.all(h[-1] == 3.0)
    assert np.all(h[:, :4] == 3.0) and np.all(h[:, n + 4:] == 3.0)
    ref = oracle.scaled_mm(d["aq"], d["wq"], d["sa"], d["sw"], True)
    assert_gemm_close(host_bf16_bits(out), ref, d["aq"], d["sa"], d["wq"], d["sw"], True)


def test_gemm_deterministic():
    d = _prepare(6, 1024, 4096, 2048, per_channel=True, rowmul=True)
    o1 = fp8.scaled_mm(d["a_q"], d["w_q"], d["s_a"], d["s_w"], True)
    o2 = fp8.scaled_mm(d["a_q"], d["w_q"], d["s_a"], d["s_w"], True)
    d2 = _prepare(6, 16, 4096, 2048, per_channel=True, rowmul=True)
    o3 = fp8.scaled_mm(d2["a_q"], d2["w_q"], d2["s_a"], d2["s_w"], True)
    o4 = fp8.scaled_mm(d2["a_q"], d2["w_q"], d2["s_a"], d2["s_w"], True)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(o3.view(torch.int16), o4.view(torch.int16))


def test_zero_activations_give_bias():
    n, k = 1030, 4096
    w = synth.weights(1, n, k); b = synth.bias(1, n)
    w_q, s_w = fp8.quant_weight(dev_bf16(w), True)
    for m in (16, 200):
        a_q, s_a = fp8.quant_dynamic(torch.zeros((m, k), dtype=torch.bfloat16, device="cuda"))
        out = fp8.scaled_mm(a_q, w_q, s_a, s_w, True, dev_bf16(b))
        torch.cuda.synchronize()
        assert np.array_equal(host_bf16_bits(out), np.broadcast_to(b, (m, n)))
