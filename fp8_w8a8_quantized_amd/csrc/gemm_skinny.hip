// Skinny-M scaled FP8 GEMM for decode (M <= 64), gfx950.
//
// "[WIP] FP8 support" (text-generation-inference PR 1484), review discussion:
// decode runs at fewer than 16 rows, wants a dedicated GEMV-like kernel, and
// must not pay for per-call packing or 16-padding.  Here the weight streams
// from HBM straight into the matrix cores' A operand, one 16-row slice of W
// per workgroup (two slices, up to 32 rows, for N of about 14300 and more), each
// byte read once; the activation rows (at most 16) are the B operand, and
// rows >= M are zeros in registers, never in memory.
//
// Accumulation: the fp8 matrix-core instruction sums each group of 8
// products with only 13 bits below the group's largest product (measured on
// gfx950), which loses small products next to large ones.  This path is
// bound by HBM, not by the matrix cores, so it converts the e4m3 codes to
// bf16 in registers (exact: every e4m3 value is a bf16 value) and uses the
// bf16 instruction v_mfma_f32_16x16x32_bf16, whose sums keep fp32-class
// precision.  HBM traffic is unchanged: one byte per weight.
//
// Memory access: one 16-byte load instruction of a wave covers 4 rows x
// 256 contiguous bytes (measured on MI355X: 16 rows x 64 bytes per
// instruction streams at about half the rate).  The matrix cores want lane l
// to hold row (l % 16) instead, so each wave transposes its 16 x 256-byte
// step through a private, XOR-swizzled LDS buffer (conflict-free on both
// the write and the read side), for the weight and for the activation rows.
// Lane l then holds row (l % 16) of each operand and, per 128-wide k half,
// bytes [16g, 16g+16) and [64+16g, 64+16g+16) with g = l / 16; both operands
// use the same lane/element -> k assignment, so products pair matching k
// whatever order the hardware sums in.
//
// The waves of a workgroup split K into 256-byte steps (contiguous ranges,
// or every fourth step for long K), run a rolling pipeline with the next
// step's loads in flight while they work on the current one, and are summed
// through LDS in a fixed order, so results do not depend on timing.  The rescale
// epilogue out = acc * (s_a * s_w[n]) + bias[n] -> bf16 is applied in the
// store ("[Kernel] Implement fallback for FP8 channelwise using
// torch._scaled_mm", description: the channelwise rescale follows the
// per-tensor GEMM; fused here instead of a separate pass).
//
// M from 17 to 64 runs a multi-block variant in which one workgroup serves
// every 16-row block of M (up to four) from each weight step, so the weight
// still streams once; larger M on this path (problems of up to 256 rows too
// small for the matrix-core GEMM's tiles, and layouts that kernel does not
// take) runs ceil(M / 64) grid rows with the blocks spread evenly over them,
// and the grid rows of one weight block share an XCD, whose L2 serves the
// repeated weight reads (so do two grid rows of fewer blocks, which replace
// one where a single row would have few workgroups).  On wide weights, M
// from 17 to 64 runs a wide variant instead: each wave owns a weight block
// over the whole of K and the workgroup loads each activation step once for
// its four blocks, so fewer activation lines pass the texture path per
// weight line.  Layouts that are not 16-byte aligned (or K % 16 != 0) use a
// byte-granular variant that loads each lane's 32 bytes directly in the
// matrix-core layout, one 16-row block of M per grid row.

#include <algorithm>
#include <atomic>

#include "device_common.h"
#include "internal.h"

namespace fp8w8a8 {

namespace {

// 32 k-bytes of one row for k step base k0s (= 128 * step): pieces at
// k0s + 16g and k0s + 64 + 16g.  VEC: rows are 16-byte aligned and
// K % 16 == 0, so a piece is either wholly inside [0, K) or wholly outside.
template <bool VEC>
__device__ __forceinline__ v8i load_frag(const uint8_t* row, int k0s, int g, int K, bool ok) {
  v8i f = {0, 0, 0, 0, 0, 0, 0, 0};
  if (!ok) return f;
  const int ka = k0s + 16 * g, kb = ka + 64;
  if constexpr (VEC) {
    if (ka < K) {
      v4i lo = *reinterpret_cast<const v4i*>(row + ka);
      f[0] = lo[0]; f[1] = lo[1]; f[2] = lo[2]; f[3] = lo[3];
    }
    if (kb < K) {
      v4i hi = *reinterpret_cast<const v4i*>(row + kb);
      f[4] = hi[0]; f[5] = hi[1]; f[6] = hi[2]; f[7] = hi[3];
    }
  } else {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int kbase = half ? kb : ka;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        uint32_t word = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int k = kbase + 4 * w + b;
          if (k < K) word |= (uint32_t)row[k] << (8 * b);
        }
        f[4 * half + w] = (int)word;
      }
    }
  }
  return f;
}

// 4 fp8 codes (one 32-bit word) of format F -> 4 bf16 values, exactly.
template <int F>
__device__ __forceinline__ void fp8x4_to_bf16(int w, bf16x8& dst, int at) {
  bf16x2 lo = fp8x2_to_bf16<F, false>(w);
  bf16x2 hi = fp8x2_to_bf16<F, true>(w);
  dst[at] = lo[0]; dst[at + 1] = lo[1]; dst[at + 2] = hi[0]; dst[at + 3] = hi[1];
}

// acc += W_frag . A_frag over 32 fp8 k-values per lane (W in format FW, A
// in FA), as four bf16 16x16x32 products (k-values 8t..8t+7 of the lane feed
// instruction t).
template <int FA, int FW>
__device__ __forceinline__ v4f mfma_fp8_as_bf16(v8i wf, v8i af, v4f acc) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    bf16x8 wb, ab;
    fp8x4_to_bf16<FW>(wf[2 * t], wb, 0);
    fp8x4_to_bf16<FW>(wf[2 * t + 1], wb, 4);
    fp8x4_to_bf16<FA>(af[2 * t], ab, 0);
    fp8x4_to_bf16<FA>(af[2 * t + 1], ab, 4);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wb, ab, acc, 0, 0, 0);
  }
  return acc;
}

// As mfma_fp8_as_bf16 with the weight fragment already converted (wb[t]:
// its k-values 8t..8t+7 as bf16), so one conversion serves several
// activation blocks.
template <int FA>
__device__ __forceinline__ v4f mfma_bf16w_fp8a(const bf16x8 (&wb)[4], v8i af, v4f acc) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    bf16x8 ab;
    fp8x4_to_bf16<FA>(af[2 * t], ab, 0);
    fp8x4_to_bf16<FA>(af[2 * t + 1], ab, 4);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wb[t], ab, acc, 0, 0, 0);
  }
  return acc;
}

// The epilogue's per-column factors, loaded at kernel start so that their
// memory latency overlaps the main loop instead of following it.  They are
// kept as loaded (no arithmetic on them until the epilogue), so no wait for
// them lands before the main loop.
struct EpiParams {
  float sw[4];
  uint32_t bias[4];
};

__device__ __forceinline__ EpiParams load_epi_params(const GemmArgs& g, int lane, int n0) {
  // Buffer loads based at the block's first column (offsets below 64 bytes
  // whatever N is); a missing bias is a resource of size 0, whose loads
  // return zeros.  No load sits under a branch.
  const int cols = min(g.N - n0, 16);
  const __amdgpu_buffer_rsrc_t rsw = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(g.per_channel ? g.s_w + n0 : g.s_w), (short)0, g.per_channel ? 4 * cols : 4, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rbias = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(g.bias ? g.bias + n0 : reinterpret_cast<const uint16_t*>(g.s_w)), (short)0, g.bias ? 2 * cols : 0,
      kRsrcWord3);
  EpiParams p;
  const int cb = 4 * (lane >> 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = min(cb + i, cols - 1);
    p.sw[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsw, g.per_channel ? 4 * c : 0, 0, 0));
    p.bias[i] = __builtin_amdgcn_raw_buffer_load_b16(rbias, 2 * c, 0, 0);
  }
  return p;
}

// Sum the waves' partial tiles through LDS in wave order and apply the
// rescale epilogue.  acc holds D[n][m] for n = n0 + 4 * (lane / 16) + i and
// m = m0 + lane % 16.
__device__ __forceinline__ void reduce_and_store(const GemmArgs& g, v4f acc, float (*red)[4][64], int nw,
                                                 int wave, int lane, int n0, int m0, const EpiParams& ep) {
#pragma unroll
  for (int i = 0; i < 4; ++i) red[wave][i][lane] = acc[i];
  __syncthreads();
  if (wave != 0) return;
  const float sa = *g.s_a;
  float sum[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float t = red[0][i][lane];
    for (int w = 1; w < nw; ++w) t += red[w][i][lane];
    sum[i] = t;
  }
  const int grp = lane >> 4;
  const int m = m0 + (lane & 15);
  if (m >= g.M || n0 >= g.N) return;
  const int nb = n0 + 4 * grp;
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = f32_to_bf16_rne(__builtin_fmaf(sum[i], sa * ep.sw[i], bf16_to_f32(ep.bias[i])));
  uint16_t* orow = g.out + (int64_t)m * g.ldo;
  if (nb + 3 < g.N && ((uintptr_t)(orow + nb) % 8) == 0) {
    uint2 v;
    v.x = o[0] | (o[1] << 16);
    v.y = o[2] | (o[3] << 16);
    *reinterpret_cast<uint2*>(orow + nb) = v;
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (nb + i < g.N) orow[nb + i] = (uint16_t)o[i];
  }
}

__device__ __forceinline__ v8i cat8(v4i lo, v4i hi) {
  v8i f;
  f[0] = lo[0]; f[1] = lo[1]; f[2] = lo[2]; f[3] = lo[3];
  f[4] = hi[0]; f[5] = hi[1]; f[6] = hi[2]; f[7] = hi[3];
  return f;
}

// Aligned layouts: rows 16-byte aligned, K % 16 == 0 and pitches below
// 2^27 bytes, so every 16-byte chunk lies wholly inside or wholly outside
// [0, K) and a 16-row block spans less than 2^31 bytes.
constexpr int64_t kMaxPitch = int64_t(1) << 27;
// 16-row blocks of M per workgroup of the multi-block kernel (one reducing
// wave per block); its activation rows (up to 64) then span less than 2^31
// bytes only for pitches below 2^25.
constexpr int kMaxSkinnyBlocks = 4;
constexpr int64_t kMaxPitchMB = int64_t(1) << 25;
// Waves per workgroup and steps in flight per wave, measured on the decode
// shapes of an 8B-class model (K = 4096 and 14336): deeper pipelines (3-8
// steps) and 8 or 16 waves were slower, a single step in flight about as
// fast for the shapes with one workgroup per CU.
constexpr int kSkinnyWaves = 4;
constexpr int kSkinnyDepth = 2;

// Rolling pipeline of depth D: before a wave transposes and multiplies step
// s it issues the loads of step s + D - 1, so D - 1 steps stay in flight
// while it computes.  Every load is an unconditional buffer load: rows past
// N or M, chunks past K and steps past the wave's range get an offset past
// the resource's end and return zeros without a memory access.  With no
// load under a branch the compiler's wait counts are exact (vmcnt of the
// steps still in flight), never a full drain.
// LDS: per wave a 2 x 4 KiB staging buffer (weight and activation step),
// then the NW x 1 KiB reduction area.
// Cache-policy bits of a buffer load (gfx950): nt, a non-temporal (streaming)
// access.
constexpr int kNonTemporal = 2;

// Compute units of the current device (looked up once per device).
int device_cus() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Rows per workgroup of the two-block kernel: the fewest workgroups per CU
// that 32-row workgroups would need, then rows (a multiple of 4) spread
// evenly over that many workgroups per CU, so every CU gets the same number.
// On the 4096 -> 28672 decode shape: 28 rows, 1024 workgroups (4 per CU),
// 21.7 against 22.2 us with 32 rows (896 workgroups, 3 or 4 per CU).
int two_block_rows(int64_t N) {
  const int64_t cus = device_cus();
  const int64_t per_cu = (N + 32 * cus - 1) / (32 * cus);
  const int64_t rows = (N + cus * per_cu - 1) / (cus * per_cu);
  return (int)std::min<int64_t>(32, (rows + 3) / 4 * 4);
}

// Two weight blocks per wave once N fills at least 7/4 x (CUs) workgroups of
// 32 rows: N >= 14305 on 256 CUs.  Measured on per-tensor GEMMs at small M
// with K = 4096 and the weights streaming from HBM: at N = 14336 (two
// 28-row workgroups per CU instead of 3 or 4 one-block workgroups) 4-12%
// faster for every M from 1 to 16; between N = 8192 and 14336 only M of 12
// and more gained (3-7%), while M of 4 and less lost 1-3%.
bool use_two_blocks(int64_t N) { return (N + 31) / 32 * 4 >= 7 * (int64_t)device_cus(); }

template <int NW, int D, bool IL, bool NT, int FA, int FW>
__global__ __launch_bounds__(NW * 64) void gemm_skinny_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t stage[NW][2][16 * 256];
  __shared__ float red[NW][4][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 15, grp = lane >> 4;
  const int n0 = blockIdx.x * 16, m0 = blockIdx.y * 16;
  const int steps = (g.K + 255) >> 8;
  // The wave's steps: interleaved across the waves (wave, wave + NW, ...),
  // so that a workgroup reads adjacent 256-byte pieces of each row together,
  // or a contiguous range per wave.
  int first, stride, count;
  if constexpr (IL) {
    first = wave;
    stride = NW;
    count = max(steps - wave + NW - 1, 0) / NW;
  } else {
    const int per = (steps + NW - 1) / NW;
    first = min(wave * per, steps);
    stride = 1;
    count = min(first + per, steps) - first;
  }
  // load mapping: instruction j covers rows 4j + lane/16, bytes 16 * (lane % 16)
  const int lr = lane >> 4, lc = (lane & 15) * 16;
  const int rows_w = min(g.N - n0, 16), rows_a = min(g.M - m0, 16);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(g.w + (int64_t)n0 * g.ldw), (short)0, (int)(rows_w * g.ldw), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(g.a + (int64_t)m0 * g.lda), (short)0, (int)(rows_a * g.lda), kRsrcWord3);
  // 32-bit offsets (pitches are below 2^27)
  const uint32_t ldw = (uint32_t)g.ldw, lda = (uint32_t)g.lda;
  uint32_t wo[4], ao[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t row = 4 * j + lr;
    wo[j] = (int)row < rows_w ? row * ldw + lc : kOutOfRange;
    ao[j] = (int)row < rows_a ? row * lda + lc : kOutOfRange;
  }
  uint8_t* LW = stage[wave][0];
  uint8_t* LA = stage[wave][1];
  const int swz_w = (lane & 15);  // chunk written by this lane (before the XOR)

  v4i wv[D][4], av[D][4];
  auto issue = [&](int slot, int i) {  // the wave's i-th step
    const int k0 = (first + i * stride) * 256;
    const bool kin = i < count && k0 + lc < g.K;
    // the step's offsets first, then its eight loads back to back (with the
    // offset arithmetic between the loads, QKV and O ran 3-6% slower)
    uint32_t ow[4], oa[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ow[j] = kin ? wo[j] + k0 : kOutOfRange;
      oa[j] = kin ? ao[j] + k0 : kOutOfRange;
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      wv[slot][j] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rw, ow[j], 0, NT ? kNonTemporal : 0));
      av[slot][j] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(ra, oa[j], 0, 0));
    }
  };
  // Issue order is pinned: the epilogue's factors first (the oldest loads,
  // so waiting for any step covers them), then the steps in order.  After
  // each issue an explicit wait leaves exactly the D - 1 younger steps in
  // flight, on every path (the compiler's own waits would otherwise follow
  // the worst order it can prove, which drains the pipeline).
  // (the offset arithmetic above stays before every load: a 64-bit
  // multiply-add it may use reads a don't-care register that could alias a
  // pending load's destination and force a drain)
  __builtin_amdgcn_sched_barrier(0);
  const EpiParams ep = load_epi_params(g, lane, n0);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int d = 0; d < D - 1; ++d) {
    issue(d, d);
    __builtin_amdgcn_sched_barrier(0);
  }
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < count; i += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      issue((d + D - 1) % D, i + d + D - 1);
      __builtin_amdgcn_s_waitcnt(wait_vmcnt(8 * (D - 1)));
      __builtin_amdgcn_sched_barrier(0);
      if (i + d < count) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int row = 4 * j + lr;
          *reinterpret_cast<v4i*>(LW + row * 256 + ((swz_w ^ row) << 4)) = wv[d][j];
          *reinterpret_cast<v4i*>(LA + row * 256 + ((swz_w ^ row) << 4)) = av[d][j];
        }
        // the same wave reads what its other lanes wrote: LDS operations of a
        // wave complete in order, so waiting for them suffices
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int c0 = t * 8 + grp, c1 = t * 8 + 4 + grp;
          const v4i wlo = *reinterpret_cast<const v4i*>(LW + r * 256 + ((c0 ^ r) << 4));
          const v4i whi = *reinterpret_cast<const v4i*>(LW + r * 256 + ((c1 ^ r) << 4));
          const v4i alo = *reinterpret_cast<const v4i*>(LA + r * 256 + ((c0 ^ r) << 4));
          const v4i ahi = *reinterpret_cast<const v4i*>(LA + r * 256 + ((c1 ^ r) << 4));
          acc = mfma_fp8_as_bf16<FA, FW>(cat8(wlo, whi), cat8(alo, ahi), acc);
        }
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        __builtin_amdgcn_wave_barrier();
      }
    }
  }
  reduce_and_store(g, acc, red, NW, wave, lane, n0, m0, ep);
}

// Two 16-row weight blocks per wave, for N of about 14300 and more with K
// below 8192 (use_two_blocks).  Each activation step a wave loads serves
// both blocks, so the texture path moves 1.5 lines per weight line instead
// of 2.  Launched with one step in flight (112 VGPRs, four waves per SIMD):
// on the 4096 -> 28672 decode shape, 23.3 -> 22.3 us against the one-block
// kernel (two steps in flight take 221 VGPRs, two waves per SIMD, and lose
// the gain).  The second block's weight step goes through the same staging
// buffer once the first block's fragments are in registers.  A workgroup
// covers wg_rows rows (a multiple of 4, at most 32); rows past those or past
// N read as zeros and are never stored.
template <int NW, int D, bool NT, int FA, int FW>
__global__ __launch_bounds__(NW * 64) void gemm_skinny2_kernel(GemmArgs g, int wg_rows) {
  __shared__ __attribute__((aligned(16))) uint8_t stage[NW][2][16 * 256];
  __shared__ float red[2][NW][4][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 15, grp = lane >> 4;
  const int n0 = blockIdx.x * wg_rows, m0 = blockIdx.y * 16;
  const int steps = (g.K + 255) >> 8;
  const int per = (steps + NW - 1) / NW;
  const int first = min(wave * per, steps);
  const int count = min(first + per, steps) - first;
  const int lr = lane >> 4, lc = (lane & 15) * 16;
  const int rows_w = min(g.N - n0, wg_rows), rows_a = min(g.M - m0, 16);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(g.w + (int64_t)n0 * g.ldw), (short)0, (int)(rows_w * g.ldw), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(g.a + (int64_t)m0 * g.lda), (short)0, (int)(rows_a * g.lda), kRsrcWord3);
  const uint32_t ldw = (uint32_t)g.ldw, lda = (uint32_t)g.lda;
  uint32_t wo[8], ao[4];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t row = 4 * j + lr;
    wo[j] = (int)row < rows_w ? row * ldw + lc : kOutOfRange;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t row = 4 * j + lr;
    ao[j] = (int)row < rows_a ? row * lda + lc : kOutOfRange;
  }
  uint8_t* LW = stage[wave][0];
  uint8_t* LA = stage[wave][1];
  const int swz_w = (lane & 15);

  v4i wv[D][8], av[D][4];
  auto issue = [&](int slot, int i) {
    const int k0 = (first + i) * 256;
    const bool kin = i < count && k0 + lc < g.K;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      wv[slot][j] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(
                                                rw, kin ? wo[j] + k0 : kOutOfRange, 0, NT ? kNonTemporal : 0));
#pragma unroll
    for (int j = 0; j < 4; ++j)
      av[slot][j] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(
                                                ra, kin ? ao[j] + k0 : kOutOfRange, 0, 0));
  };
  __builtin_amdgcn_sched_barrier(0);
  const EpiParams ep0 = load_epi_params(g, lane, min(n0, g.N - 1));
  const EpiParams ep1 = load_epi_params(g, lane, min(n0 + 16, g.N - 1));
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int d = 0; d < D - 1; ++d) {
    issue(d, d);
    __builtin_amdgcn_sched_barrier(0);
  }
  v4f acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < count; i += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      issue((d + D - 1) % D, i + d + D - 1);
      __builtin_amdgcn_s_waitcnt(wait_vmcnt(12 * (D - 1)));
      __builtin_amdgcn_sched_barrier(0);
      if (i + d < count) {
        // block 0 and the activation step
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int row = 4 * j + lr;
          *reinterpret_cast<v4i*>(LW + row * 256 + ((swz_w ^ row) << 4)) = wv[d][j];
          *reinterpret_cast<v4i*>(LA + row * 256 + ((swz_w ^ row) << 4)) = av[d][j];
        }
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        __builtin_amdgcn_wave_barrier();
        v8i afr[2], wfr[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int c0 = t * 8 + grp, c1 = t * 8 + 4 + grp;
          wfr[t] = cat8(*reinterpret_cast<const v4i*>(LW + r * 256 + ((c0 ^ r) << 4)),
                        *reinterpret_cast<const v4i*>(LW + r * 256 + ((c1 ^ r) << 4)));
          afr[t] = cat8(*reinterpret_cast<const v4i*>(LA + r * 256 + ((c0 ^ r) << 4)),
                        *reinterpret_cast<const v4i*>(LA + r * 256 + ((c1 ^ r) << 4)));
        }
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        __builtin_amdgcn_wave_barrier();
        // block 1 into the same staging buffer (block 0's fragments are in registers)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int row = 4 * j + lr;
          *reinterpret_cast<v4i*>(LW + row * 256 + ((swz_w ^ row) << 4)) = wv[d][4 + j];
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) acc0 = mfma_fp8_as_bf16<FA, FW>(wfr[t], afr[t], acc0);
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int c0 = t * 8 + grp, c1 = t * 8 + 4 + grp;
          const v8i w1 = cat8(*reinterpret_cast<const v4i*>(LW + r * 256 + ((c0 ^ r) << 4)),
                              *reinterpret_cast<const v4i*>(LW + r * 256 + ((c1 ^ r) << 4)));
          acc1 = mfma_fp8_as_bf16<FA, FW>(w1, afr[t], acc1);
        }
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        __builtin_amdgcn_wave_barrier();
      }
    }
  }
  GemmArgs gs = g;  // stores end at this workgroup's last row
  gs.N = min(g.N, n0 + wg_rows);
  reduce_and_store(gs, acc0, red[0], NW, wave, lane, n0, m0, ep0);
  reduce_and_store(gs, acc1, red[1], NW, wave, lane, n0 + 16, m0, ep1);
}

// MB 16-row blocks of M per workgroup (M from 17 to 64 in one grid row,
// larger M in grid rows of 16 * MB): each weight step a wave loads serves
// every block, so the weight streams from HBM once per 16 * MB rows instead
// of once per 16.  The pipeline is the one-block kernel's; each block has its
// own activation staging buffer and accumulator, and the weight step is
// transposed and its fragments read once for all blocks.  After the main
// loop each wave parks its partial tiles in its own staging area and wave b
// reduces and stores block b.
template <int NW, int D, int MB, bool IL, bool NT, int FA, int FW>
__global__ __launch_bounds__(NW * 64) void gemm_skinny_mb_kernel(GemmArgs g) {
  static_assert(MB >= 1 && MB <= NW, "one reducing wave per block");
  __shared__ __attribute__((aligned(16))) uint8_t stage[NW][1 + MB][16 * 256];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 15, grp = lane >> 4;
  // Workgroups are dealt to the 8 XCDs in dispatch order (x fastest).  The
  // linear id is taken apart so that the grid rows of M of one weight block
  // come 8 ids apart: the same XCD at about the same time, so the weight
  // block streams from HBM once and that XCD's L2 serves the other rows.
  const uint32_t tn = gridDim.x, tm = gridDim.y;
  const uint32_t id = blockIdx.x + blockIdx.y * tn;
  const uint32_t group = id / (8 * tm), rem = id - group * (8 * tm);
  const uint32_t width = min(8u, tn - group * 8);  // weight blocks in this group
  const int n0 = (int)(group * 8 + rem % width) * 16, m0 = (int)(rem / width) * (16 * MB);
  const int steps = (g.K + 255) >> 8;
  int first, stride, count;
  if constexpr (IL) {
    first = wave;
    stride = NW;
    count = max(steps - wave + NW - 1, 0) / NW;
  } else {
    const int per = (steps + NW - 1) / NW;
    first = min(wave * per, steps);
    stride = 1;
    count = min(first + per, steps) - first;
  }
  const int lr = lane >> 4, lc = (lane & 15) * 16;
  const int rows_w = min(g.N - n0, 16), rows_a = min(g.M - m0, 16 * MB);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(g.w + (int64_t)n0 * g.ldw), (short)0, (int)(rows_w * g.ldw), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(g.a + (int64_t)m0 * g.lda), (short)0, (int)(rows_a * g.lda), kRsrcWord3);
  const uint32_t ldw = (uint32_t)g.ldw, lda = (uint32_t)g.lda;
  uint32_t wo[4], ao[MB][4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t row = 4 * j + lr;
    wo[j] = (int)row < rows_w ? row * ldw + lc : kOutOfRange;
#pragma unroll
    for (int b = 0; b < MB; ++b) {
      const uint32_t rowa = 16 * b + row;
      ao[b][j] = (int)rowa < rows_a ? rowa * lda + lc : kOutOfRange;
    }
  }
  uint8_t* LW = stage[wave][0];
  const int swz_w = (lane & 15);

  v4i wv[D][4], av[D][MB][4];
  auto issue = [&](int slot, int i) {  // the wave's i-th step
    const int k0 = (first + i * stride) * 256;
    const bool kin = i < count && k0 + lc < g.K;
    uint32_t ow[4], oa[MB][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ow[j] = kin ? wo[j] + k0 : kOutOfRange;
#pragma unroll
      for (int b = 0; b < MB; ++b) oa[b][j] = kin ? ao[b][j] + k0 : kOutOfRange;
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      wv[slot][j] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rw, ow[j], 0, NT ? kNonTemporal : 0));
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        av[slot][b][j] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(ra, oa[b][j], 0, 0));
  };
  constexpr int kLoads = 4 + 4 * MB;  // per step
  __builtin_amdgcn_sched_barrier(0);
  const EpiParams ep = load_epi_params(g, lane, n0);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int d = 0; d < D - 1; ++d) {
    issue(d, d);
    __builtin_amdgcn_sched_barrier(0);
  }
  v4f acc[MB];
#pragma unroll
  for (int b = 0; b < MB; ++b) acc[b] = v4f{0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < count; i += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      issue((d + D - 1) % D, i + d + D - 1);
      __builtin_amdgcn_s_waitcnt(wait_vmcnt(kLoads * (D - 1)));
      __builtin_amdgcn_sched_barrier(0);
      if (i + d < count) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int row = 4 * j + lr;
          *reinterpret_cast<v4i*>(LW + row * 256 + ((swz_w ^ row) << 4)) = wv[d][j];
#pragma unroll
          for (int b = 0; b < MB; ++b)
            *reinterpret_cast<v4i*>(stage[wave][1 + b] + row * 256 + ((swz_w ^ row) << 4)) = av[d][b][j];
        }
        // the same wave reads what its other lanes wrote: LDS operations of a
        // wave complete in order, so waiting for them suffices
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int c0 = t * 8 + grp, c1 = t * 8 + 4 + grp;
          const v8i wf = cat8(*reinterpret_cast<const v4i*>(LW + r * 256 + ((c0 ^ r) << 4)),
                              *reinterpret_cast<const v4i*>(LW + r * 256 + ((c1 ^ r) << 4)));
          bf16x8 wb[4];  // the weight fragment converted once for every block
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            fp8x4_to_bf16<FW>(wf[2 * u], wb[u], 0);
            fp8x4_to_bf16<FW>(wf[2 * u + 1], wb[u], 4);
          }
#pragma unroll
          for (int b = 0; b < MB; ++b) {
            const uint8_t* LA = stage[wave][1 + b];
            const v8i af = cat8(*reinterpret_cast<const v4i*>(LA + r * 256 + ((c0 ^ r) << 4)),
                                *reinterpret_cast<const v4i*>(LA + r * 256 + ((c1 ^ r) << 4)));
            acc[b] = mfma_bf16w_fp8a<FA>(wb, af, acc[b]);
          }
        }
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        __builtin_amdgcn_wave_barrier();
      }
    }
  }
  // partial tiles into this wave's own staging area (no other wave touches
  // it), then wave b sums block b over the waves in wave order and stores it
  float* mine = reinterpret_cast<float*>(stage[wave][0]);
#pragma unroll
  for (int b = 0; b < MB; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) mine[(b * 4 + i) * 64 + lane] = acc[b][i];
  __syncthreads();
  if (wave >= MB) return;
  const int b = wave;
  float sum[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float t = reinterpret_cast<const float*>(stage[0][0])[(b * 4 + i) * 64 + lane];
    for (int w = 1; w < NW; ++w) t += reinterpret_cast<const float*>(stage[w][0])[(b * 4 + i) * 64 + lane];
    sum[i] = t;
  }
  const float sa = *g.s_a;
  const int m = m0 + 16 * b + (lane & 15);
  if (m >= g.M) return;
  const int nb = n0 + 4 * grp;
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = f32_to_bf16_rne(__builtin_fmaf(sum[i], sa * ep.sw[i], bf16_to_f32(ep.bias[i])));
  uint16_t* orow = g.out + (int64_t)m * g.ldo;
  if (nb + 3 < g.N && ((uintptr_t)(orow + nb) % 8) == 0) {
    uint2 v;
    v.x = o[0] | (o[1] << 16);
    v.y = o[2] | (o[3] << 16);
    *reinterpret_cast<uint2*>(orow + nb) = v;
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (nb + i < g.N) orow[nb + i] = (uint16_t)o[i];
  }
}

// Wide weights at small M: each of the 4 waves owns its own 16-row weight
// block (64 rows per workgroup) and walks the whole of K, so no partial
// tiles are summed across waves.  The activation rows of a step are loaded
// once per workgroup -- wave b loads the step of M block b -- into a shared
// LDS area double-buffered by step parity, and every wave multiplies its
// weight block with all of them: per weight line the texture path moves
// MB / 4 activation lines instead of MB (the multi-block kernel) or 1 / 2
// (the two-block kernel).  One workgroup barrier per step orders the shared
// area: a step's blocks are complete at it, and a wave writes a buffer again
// two steps later only after every wave has passed the barrier that follows
// its reads of it.  Waves whose block starts past N load nothing (a resource
// of size 0) and store nothing.
template <int MB, int D, bool NT, int FA, int FW>
__global__ __launch_bounds__(256) void gemm_skinny_wide_kernel(GemmArgs g) {
  static_assert(MB >= 1 && MB <= 4, "one loading wave per block of M");
  __shared__ __attribute__((aligned(16))) uint8_t wstage[4][16 * 256];
  __shared__ __attribute__((aligned(16))) uint8_t astage[2][MB][16 * 256];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 15, grp = lane >> 4;
  const int n0 = blockIdx.x * 64 + wave * 16, m0 = blockIdx.y * (16 * MB);
  const int steps = (g.K + 255) >> 8;
  const int lr = lane >> 4, lc = (lane & 15) * 16;
  const int rows_w = max(min(g.N - n0, 16), 0), rows_a = min(g.M - m0, 16 * MB);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(g.w + (int64_t)min(n0, g.N - 1) * g.ldw), (short)0, (int)(rows_w * g.ldw), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(g.a + (int64_t)m0 * g.lda), (short)0, (int)(rows_a * g.lda), kRsrcWord3);
  const uint32_t ldw = (uint32_t)g.ldw, lda = (uint32_t)g.lda;
  // this wave's weight rows, and the rows of its M block (waves >= MB load none)
  uint32_t wo[4], ao[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t row = 4 * j + lr;
    wo[j] = (int)row < rows_w ? row * ldw + lc : kOutOfRange;
    const uint32_t rowa = 16 * wave + row;
    ao[j] = wave < MB && (int)rowa < rows_a ? rowa * lda + lc : kOutOfRange;
  }
  uint8_t* LW = wstage[wave];
  const int swz_w = (lane & 15);

  v4i wv[D][4], av[D][4];
  auto issue = [&](int slot, int i) {  // step i
    const int k0 = i * 256;
    const bool kin = i < steps && k0 + lc < g.K;
    uint32_t ow[4], oa[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ow[j] = kin ? wo[j] + k0 : kOutOfRange;
      oa[j] = kin ? ao[j] + k0 : kOutOfRange;
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      wv[slot][j] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rw, ow[j], 0, NT ? kNonTemporal : 0));
#pragma unroll
    for (int j = 0; j < 4; ++j)
      av[slot][j] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(ra, oa[j], 0, 0));
  };
  __builtin_amdgcn_sched_barrier(0);
  const EpiParams ep = load_epi_params(g, lane, min(n0, g.N - 1));
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int d = 0; d < D - 1; ++d) {
    issue(d, d);
    __builtin_amdgcn_sched_barrier(0);
  }
  v4f acc[MB];
#pragma unroll
  for (int b = 0; b < MB; ++b) acc[b] = v4f{0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < steps; i += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      issue((d + D - 1) % D, i + d + D - 1);
      __builtin_amdgcn_s_waitcnt(wait_vmcnt(8 * (D - 1)));
      __builtin_amdgcn_sched_barrier(0);
      if (i + d < steps) {  // the same for every wave of the workgroup
        uint8_t(*const AS)[16 * 256] = astage[(i + d) & 1];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int row = 4 * j + lr;
          *reinterpret_cast<v4i*>(LW + row * 256 + ((swz_w ^ row) << 4)) = wv[d][j];
          if (wave < MB) *reinterpret_cast<v4i*>(AS[wave] + row * 256 + ((swz_w ^ row) << 4)) = av[d][j];
        }
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        __syncthreads();
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int c0 = t * 8 + grp, c1 = t * 8 + 4 + grp;
          const v8i wf = cat8(*reinterpret_cast<const v4i*>(LW + r * 256 + ((c0 ^ r) << 4)),
                              *reinterpret_cast<const v4i*>(LW + r * 256 + ((c1 ^ r) << 4)));
          bf16x8 wb[4];  // the weight fragment converted once for every block
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            fp8x4_to_bf16<FW>(wf[2 * u], wb[u], 0);
            fp8x4_to_bf16<FW>(wf[2 * u + 1], wb[u], 4);
          }
#pragma unroll
          for (int b = 0; b < MB; ++b) {
            const uint8_t* LA = AS[b];
            const v8i af = cat8(*reinterpret_cast<const v4i*>(LA + r * 256 + ((c0 ^ r) << 4)),
                                *reinterpret_cast<const v4i*>(LA + r * 256 + ((c1 ^ r) << 4)));
            acc[b] = mfma_bf16w_fp8a<FA>(wb, af, acc[b]);
          }
        }
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        __builtin_amdgcn_wave_barrier();
      }
    }
  }
  if (n0 >= g.N) return;
  const float sa = *g.s_a;
  const int nb = n0 + 4 * grp;
#pragma unroll
  for (int b = 0; b < MB; ++b) {
    const int m = m0 + 16 * b + (lane & 15);
    if (m >= g.M) break;
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o[i] = f32_to_bf16_rne(__builtin_fmaf(acc[b][i], sa * ep.sw[i], bf16_to_f32(ep.bias[i])));
    uint16_t* orow = g.out + (int64_t)m * g.ldo;
    if (nb + 3 < g.N && ((uintptr_t)(orow + nb) % 8) == 0) {
      uint2 v;
      v.x = o[0] | (o[1] << 16);
      v.y = o[2] | (o[3] << 16);
      *reinterpret_cast<uint2*>(orow + nb) = v;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (nb + i < g.N) orow[nb + i] = (uint16_t)o[i];
    }
  }
}

template <int NW, int U, bool VEC, int FA, int FW>
__global__ __launch_bounds__(NW * 64) void gemm_skinny_generic_kernel(GemmArgs g) {
  __shared__ float red[NW][4][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 15, grp = lane >> 4;
  const int n0 = blockIdx.x * 16, m0 = blockIdx.y * 16;
  const bool n_ok = n0 + r < g.N, m_ok = m0 + r < g.M;
  const uint8_t* wrow = g.w + (int64_t)(n_ok ? n0 + r : 0) * g.ldw;
  const uint8_t* arow = g.a + (int64_t)(m_ok ? m0 + r : 0) * g.lda;
  const int ks = (g.K + 127) >> 7;

  const EpiParams ep = load_epi_params(g, lane, n0);
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = wave; s0 < ks; s0 += NW * U) {
    v8i wf[U], af[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = s0 + u * NW;
      wf[u] = load_frag<VEC>(wrow, s * 128, grp, g.K, n_ok && s < ks);
      af[u] = load_frag<VEC>(arow, s * 128, grp, g.K, m_ok && s < ks);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc = mfma_fp8_as_bf16<FA, FW>(wf[u], af[u], acc);
  }

  reduce_and_store(g, acc, red, NW, wave, lane, n0, m0, ep);
}

template <int NW, int FA, int FW>
hipError_t launch_generic(const GemmArgs& g, dim3 grid, hipStream_t stream) {
  constexpr int U = NW >= 16 ? 4 : 8;  // 16 waves leave 128 VGPRs per lane
  gemm_skinny_generic_kernel<NW, U, false, FA, FW><<<grid, NW * 64, 0, stream>>>(g);
  return hipGetLastError();
}

// Rows of M per grid row of the multi-block kernel.
// The 16-row blocks of M are spread evenly over the ceil(M / 64) grid rows
// (65 rows: two grid rows of 3 blocks, not 4 + 4), so no grid row runs
// blocks that lie wholly past M.  From 33 to 64 rows two grid rows of fewer
// blocks replace one where a single row leaves the GPU short of workgroups:
// N / 16 at most CUs / 2, or four blocks with N / 16 between CUs and
// 2 x CUs.  (Per-channel GEMMs, weights from HBM, alternating runs: N = 1030
// at M = 33-64 9.0-10.3 -> 7.1-7.4 us; N = 6144 at M = 56-64 16.3-16.8 ->
// 14.0-14.6 us with K = 4096 and 48.2-48.8 -> 40.5-41.6 us with K = 14336;
// elsewhere two rows lost up to 39%, e.g. K = 14336, N = 4096.)
int skinny_rows_per_grid_row(const GemmArgs& g) {
  const int blocks = (g.M + 15) / 16;
  int grid_rows = (blocks + kMaxSkinnyBlocks - 1) / kMaxSkinnyBlocks;
  const int64_t wgs = ((int64_t)g.N + 15) / 16, cus = device_cus();
  if (grid_rows == 1 && blocks > 2 && (wgs <= cus / 2 || (blocks == 4 && wgs > cus && wgs < 2 * cus)))
    grid_rows = 2;
  return 16 * ((blocks + grid_rows - 1) / grid_rows);
}

template <int MB, int FA, int FW>
hipError_t launch_mb(const GemmArgs& g, hipStream_t stream) {
  const bool il = (g.K + 255) / 256 >= 32;
  const bool nt = (int64_t)g.N * g.K >= (int64_t(32) << 20);
  const dim3 grid((unsigned)((g.N + 15) / 16), (unsigned)((g.M + 16 * MB - 1) / (16 * MB)));
  const dim3 block(kSkinnyWaves * 64);
  if (il && nt)
    gemm_skinny_mb_kernel<kSkinnyWaves, kSkinnyDepth, MB, true, true, FA, FW><<<grid, block, 0, stream>>>(g);
  else if (il)
    gemm_skinny_mb_kernel<kSkinnyWaves, kSkinnyDepth, MB, true, false, FA, FW><<<grid, block, 0, stream>>>(g);
  else if (nt)
    gemm_skinny_mb_kernel<kSkinnyWaves, kSkinnyDepth, MB, false, true, FA, FW><<<grid, block, 0, stream>>>(g);
  else
    gemm_skinny_mb_kernel<kSkinnyWaves, kSkinnyDepth, MB, false, false, FA, FW><<<grid, block, 0, stream>>>(g);
  return hipGetLastError();
}

template <int FA, int FW>
hipError_t launch_skinny_mb(const GemmArgs& g, hipStream_t stream) {
  switch (skinny_rows_per_grid_row(g) / 16) {
    case 2: return launch_mb<2, FA, FW>(g, stream);
    case 3: return launch_mb<3, FA, FW>(g, stream);
    default: return launch_mb<4, FA, FW>(g, stream);
  }
}

// The wide kernel (16 < M <= 64) where it measured faster than the
// multi-block kernel: M > 32 with N >= 56 x CUs, or M > 16 with N >= 112 x
// CUs (N / 64 workgroups, one per CU or more).  Per-channel GEMMs with
// K = 4096, weights streaming from HBM, alternating runs: N = 14336 at
// M = 33-64 8-19% faster (64 rows: 29.9 -> 24.3 us), N = 28672 at M = 17-48
// 7-22% faster, N = 57344 5-26%; at N = 8192 (128 workgroups) 30-58%
// slower, at N = 14336 with M <= 32 and N = 24576 with M = 17 within 5%
// either way.  Two steps in flight beat three.
bool use_wide(int64_t M, int64_t N) {
  const int64_t cus = device_cus();
  return M > 16 && M <= 64 && ((M > 32 && N >= 56 * cus) || N >= 112 * cus);
}
constexpr int kWideDepth = 2;

template <int MB, int FA, int FW>
hipError_t launch_wide_mb(const GemmArgs& g, hipStream_t stream) {
  const bool nt = (int64_t)g.N * g.K >= (int64_t(32) << 20);
  const dim3 grid((unsigned)((g.N + 63) / 64), 1);
  if (nt)
    gemm_skinny_wide_kernel<MB, kWideDepth, true, FA, FW><<<grid, 256, 0, stream>>>(g);
  else
    gemm_skinny_wide_kernel<MB, kWideDepth, false, FA, FW><<<grid, 256, 0, stream>>>(g);
  return hipGetLastError();
}

template <int FA, int FW>
hipError_t launch_wide(const GemmArgs& g, hipStream_t stream) {
  switch ((g.M + 15) / 16) {
    case 1: return launch_wide_mb<1, FA, FW>(g, stream);
    case 2: return launch_wide_mb<2, FA, FW>(g, stream);
    case 3: return launch_wide_mb<3, FA, FW>(g, stream);
    default: return launch_wide_mb<4, FA, FW>(g, stream);
  }
}

template <int FA, int FW>
hipError_t launch_skinny(const GemmArgs& g, hipStream_t stream) {
  const bool aligned = ((uintptr_t)g.a % 16 == 0) && ((uintptr_t)g.w % 16 == 0) && (g.lda % 16 == 0) &&
                       (g.ldw % 16 == 0) && (g.K % 16 == 0) && g.lda < kMaxPitch && g.ldw < kMaxPitch &&
                       g.N < (1 << 29) && (g.M <= 16 || g.lda < kMaxPitchMB);
  const int64_t tiles_n = ((int64_t)g.N + 15) / 16, tiles_m = ((int64_t)g.M + 15) / 16;  // N may come near 2^31
  dim3 grid((unsigned)tiles_n, (unsigned)tiles_m);
  if (aligned && use_wide(g.M, g.N)) return launch_wide<FA, FW>(g, stream);
  if (aligned && g.M > 16) return launch_skinny_mb<FA, FW>(g, stream);
  if (aligned) {
    // Interleaved steps for long K (>= 8192), contiguous ranges otherwise;
    // weights of 32 MiB and more streamed with non-temporal loads.  Each
    // choice was the faster one on the decode shapes of an 8B-class model
    // with weights streaming from HBM: the non-temporal hint took gate_up
    // (112 MiB) from 25.9 to 23.2 us and down (56 MiB) from 14.0 to 13.4 us,
    // but slowed QKV (24 MiB) and O (16 MiB) by 0.4-1 us.
    const bool il = (g.K + 255) / 256 >= 32;
    const bool nt = (int64_t)g.N * g.K >= (int64_t(32) << 20);
    const dim3 block(kSkinnyWaves * 64);
    if (!il && use_two_blocks(g.N)) {
      const int rw = two_block_rows(g.N);
      const dim3 grid2((unsigned)((g.N + rw - 1) / rw), (unsigned)tiles_m);
      if (nt)
        gemm_skinny2_kernel<kSkinnyWaves, 1, true, FA, FW><<<grid2, block, 0, stream>>>(g, rw);
      else
        gemm_skinny2_kernel<kSkinnyWaves, 1, false, FA, FW><<<grid2, block, 0, stream>>>(g, rw);
      return hipGetLastError();
    }
    if (il && nt)
      gemm_skinny_kernel<kSkinnyWaves, kSkinnyDepth, true, true, FA, FW><<<grid, block, 0, stream>>>(g);
    else if (il)
      gemm_skinny_kernel<kSkinnyWaves, kSkinnyDepth, true, false, FA, FW><<<grid, block, 0, stream>>>(g);
    else if (nt)
      gemm_skinny_kernel<kSkinnyWaves, kSkinnyDepth, false, true, FA, FW><<<grid, block, 0, stream>>>(g);
    else
      gemm_skinny_kernel<kSkinnyWaves, kSkinnyDepth, false, false, FA, FW><<<grid, block, 0, stream>>>(g);
    return hipGetLastError();
  }
  const int64_t tiles = tiles_n * tiles_m;
  const int ks = (g.K + 127) / 128;
  int nw = tiles >= 256 ? 4 : (tiles >= 128 ? 8 : 16);
  while (nw > 1 && nw > ks) nw >>= 1;
  switch (nw) {
    case 16: return launch_generic<16, FA, FW>(g, grid, stream);
    case 8: return launch_generic<8, FA, FW>(g, grid, stream);
    case 4: return launch_generic<4, FA, FW>(g, grid, stream);
    case 2: return launch_generic<2, FA, FW>(g, grid, stream);
    default: return launch_generic<1, FA, FW>(g, grid, stream);
  }
}

}  // namespace

hipError_t launch_gemm_skinny(const GemmArgs& g, hipStream_t stream) {
  if (g.fmt_a == kE5M2)
    return g.fmt_w == kE5M2 ? launch_skinny<kE5M2, kE5M2>(g, stream) : launch_skinny<kE5M2, kE4M3>(g, stream);
  return g.fmt_w == kE5M2 ? launch_skinny<kE4M3, kE5M2>(g, stream) : launch_skinny<kE4M3, kE4M3>(g, stream);
}

}  // namespace fp8w8a8
