// Scaled FP8 GEMM on the gfx950 matrix cores for M > 16 (prefill), with the
// rescale epilogue fused into the store.
//
// out[m, n] = bf16( sum_k A[m, k] * W[n, k] * (s_a * s_w[n]) + bias[n] ):
// the W8A8 linear of "Prototype FP8Linear W8A8 runtime quantization"
// (opening post), with the channelwise rescale that "[Kernel] Implement
// fallback for FP8 channelwise using torch._scaled_mm" (description) runs
// as a separate pass after the per-tensor GEMM applied here in the store.
//
// Design for CDNA4:
//   * 256 x 256 output tile per workgroup, 128 k per step; 4 waves, each
//     owning a 128 x 128 quarter as 4 x 4 blocks of
//     v_mfma_f32_32x32x64_f8f6f4 (256 fp32 accumulators per lane).
//   * Both operands are K-contiguous ([M, K] and [N, K]), which is the
//     matrix cores' native operand layout: every lane reads 32 contiguous
//     k-bytes of one row, so no transposition is needed anywhere.
//   * Global -> LDS directly (buffer_load ... lds, no staging registers),
//     double-buffered (2 x 64 KiB); the next step's loads are in flight
//     while the current step's products run.  Out-of-range lanes (rows past
//     M or N, k past K) return zeros, so edge tiles need no branches and k
//     tails add nothing.  Each k step reads all its fragments first and
//     interleaves the remaining LDS reads and the next step's loads with
//     the matrix products (scheduling barriers).
//   * LDS rows are 128 bytes; the 16-byte chunk c of row r is stored at
//     position c ^ (r & 7), so the 8 rows that 8 consecutive lanes read land
//     in 8 different bank groups.
//   * Tile order: the hardware deals workgroups round-robin to the 8 XCDs;
//     the id is remapped so each XCD owns a contiguous run of tiles, and
//     that run walks groups of 8 tile-rows, so the A and W panels a group
//     touches stay in that XCD's L2.
//   * The accumulation is per-tile, in a fixed order: results are
//     deterministic.
//   * Two accumulation modes (template EXACT).  The fp8 instruction
//     (v_mfma_f32_32x32x64_f8f6f4) sums each group of 8 products keeping
//     only 13 bits below the group's largest product (measured on gfx950):
//     twice the throughput, but small products beside large ones are
//     truncated.  EXACT converts each fp8 fragment to bf16 in registers
//     (exact: every e4m3 value is a bf16 value) and runs
//     v_mfma_f32_32x32x16_bf16, whose sums keep fp32-class precision; the
//     LDS tiles, the loads and the HBM traffic are the same in both modes.

#include "device_common.h"
#include "internal.h"

namespace fp8w8a8 {

namespace {

constexpr int BM = 256, BN = 256, BK = 128;
constexpr int kThreads = 256;
constexpr int kOperandBytes = BM * BK;  // 32 KiB per operand per stage
constexpr int kStageBytes = 2 * kOperandBytes;
constexpr int kGroupM = 8;
constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format (gfx9)

__device__ __forceinline__ int lds_off(int row, int chunk) { return row * BK + ((chunk ^ (row & 7)) << 4); }

__device__ __forceinline__ v8i read_frag(const uint8_t* base, int row, int chunk) {
  const v4i lo = *reinterpret_cast<const v4i*>(base + lds_off(row, chunk));
  const v4i hi = *reinterpret_cast<const v4i*>(base + lds_off(row, chunk + 1));
  v8i f;
  f[0] = lo[0]; f[1] = lo[1]; f[2] = lo[2]; f[3] = lo[3];
  f[4] = hi[0]; f[5] = hi[1]; f[6] = hi[2]; f[7] = hi[3];
  return f;
}

// 4 e4m3 codes -> 4 bf16 values of dst starting at element `at` (exact).
__device__ __forceinline__ void e4m3x4_to_bf16(int w, bf16x8& dst, int at) {
  bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  dst[at] = lo[0]; dst[at + 1] = lo[1]; dst[at + 2] = hi[0]; dst[at + 3] = hi[1];
}

__device__ __forceinline__ bf16x8 slice_bf16(const v8i& f, int t) {
  bf16x8 b;
  e4m3x4_to_bf16(f[2 * t], b, 0);
  e4m3x4_to_bf16(f[2 * t + 1], b, 4);
  return b;
}

template <bool EXACT>
__global__ __launch_bounds__(kThreads, 1) void gemm_mfma_kernel(GemmArgs g, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * kStageBytes];

  // ---- tile coordinates: XCD-contiguous, then grouped along M
  int b = blockIdx.x;
  const int T = tiles_m * tiles_n;
  if ((T & 7) == 0) b = (b & 7) * (T >> 3) + (b >> 3);
  const int per_group = kGroupM * tiles_n;
  const int first_m = (b / per_group) * kGroupM;
  const int gm = min(tiles_m - first_m, kGroupM);
  const int tm = first_m + (b % per_group) % gm;
  const int tn = (b % per_group) / gm;
  const int m0 = tm * BM, n0 = tn * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- buffer resources based at the tile's first row
  const int rows_a = min(BM, g.M - m0), rows_w = min(BN, g.N - n0);
  const uint8_t* abase = g.a + (int64_t)m0 * g.lda;
  const uint8_t* wbase = g.w + (int64_t)n0 * g.ldw;
  const uint32_t nrec_a = (uint32_t)((int64_t)(rows_a - 1) * g.lda + g.K);
  const uint32_t nrec_w = (uint32_t)((int64_t)(rows_w - 1) * g.ldw + g.K);
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc((void*)abase, (short)0, (int)nrec_a, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc((void*)wbase, (short)0, (int)nrec_w, kRsrcWord3);

  // ---- loader: buffer_load_dwordx4 ... lds.  Each wave instruction fills
  // one dense 1 KiB LDS block (8 rows x 128 bytes, lane i -> bytes 16i ..
  // 16i+15, the block's base in M0); the XOR swizzle is applied by choosing
  // which global chunk each lane fetches.  Block b of an operand is loaded
  // by wave b / 8.  Out-of-range lanes (rows past M or N, k past K, or a
  // whole step past the end) return zeros.
  uint32_t dvoff_a[8], dvoff_w[8];
  const int drow_in_blk = lane >> 3, dphys = lane & 7;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = (wave * 8 + i) * 8 + drow_in_blk;
    const int c = dphys ^ (row & 7);
    dvoff_a[i] = row < rows_a ? (uint32_t)(row * g.lda + c * 16) : kOutOfRange;
    dvoff_w[i] = row < rows_w ? (uint32_t)(row * g.ldw + c * 16) : kOutOfRange;
  }
  const int dchunk_k = (dphys ^ drow_in_blk) * 16;  // row & 7 == drow_in_blk
  auto dma = [&](int stage, int k0, bool step_valid) {
    const bool kin = step_valid && k0 + dchunk_k < g.K;
    uint8_t* As = smem + stage * kStageBytes;
    uint8_t* Ws = As + kOperandBytes;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int blk = __builtin_amdgcn_readfirstlane(wave * 8 + i);
      const uint32_t oa = (kin && dvoff_a[i] != kOutOfRange) ? dvoff_a[i] + k0 : kOutOfRange;
      const uint32_t ow = (kin && dvoff_w[i] != kOutOfRange) ? dvoff_w[i] + k0 : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (__attribute__((address_space(3))) void*)(As + blk * 1024), 16,
                                               (int)oa, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (__attribute__((address_space(3))) void*)(Ws + blk * 1024), 16,
                                               (int)ow, 0, 0, 0);
    }
  };

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int KT = (g.K + BK - 1) / BK;
  const int frow = lane & 31;          // operand row within a 32-row block
  const int fchunk = (lane >> 5) * 2;  // first of the lane's two chunks

  dma(0, 0, true);
  for (int kt = 0; kt < KT; ++kt) {
    __builtin_amdgcn_s_waitcnt(kWaitVm0);  // this wave's loads for stage kt landed
    __syncthreads();                       // ... and every other wave's
    // next stage (an all-zero load into the idle buffer after the last
    // step, which keeps the loop body one basic block for the scheduler)
    dma((kt + 1) & 1, (kt + 1) * BK, kt + 1 < KT);
    const uint8_t* As = smem + (kt & 1) * kStageBytes;
    const uint8_t* Ws = As + kOperandBytes;
    // all fragments of this k step first (both 64-wide halves), so the
    // second half's LDS latency hides under the first half's products
    v8i wf[2][4], af[2][4];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int i = 0; i < 4; ++i) wf[ks][i] = read_frag(Ws, wn * 128 + i * 32 + frow, ks * 4 + fchunk);
#pragma unroll
      for (int j = 0; j < 4; ++j) af[ks][j] = read_frag(As, wm * 128 + j * 32 + frow, ks * 4 + fchunk);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      if constexpr (!EXACT) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wf[ks][i], af[ks][j], acc[i][j], 0, 0, 0,
                                                                         0, 0, 0);
      } else {
        // the lane's 32 k-values in four slices of 8 (same slicing for both
        // operands), one bf16 32x32x16 product per slice
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          bf16x8 wb[4], ab[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) wb[i] = slice_bf16(wf[ks][i], t);
#pragma unroll
          for (int j = 0; j < 4; ++j) ab[j] = slice_bf16(af[ks][j], t);
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wb[i], ab[j], acc[i][j], 0, 0, 0);
        }
      }
    }
    if constexpr (!EXACT) {
      // issue order: the first half's 16 LDS reads, then one product per
      // LDS read of the second half, then one product per load of the next
      // stage, then the rest
      __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
    }
  }

  // ---- epilogue.  acc[i][j] = D[n][m] for the 32x32 block (i: n, j: m):
  // lane holds m = lane % 32 and, in registers 4q..4q+3, the four
  // consecutive columns n = 8q + 4 * (lane / 32) + 0..3.
  const float sa = *g.s_a;
  const bool vec_out = ((uintptr_t)g.out % 8 == 0) && (g.ldo % 4 == 0);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int nb = n0 + wn * 128 + i * 32 + 8 * q + 4 * (lane >> 5);
      float sc[4], bs[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int n = min(nb + e, g.N - 1);
        sc[e] = sa * (g.per_channel ? g.s_w[n] : g.s_w[0]);
        bs[e] = g.bias ? bf16_to_f32(g.bias[n]) : 0.0f;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int m = m0 + wm * 128 + j * 32 + (lane & 31);
        if (m >= g.M) continue;
        uint32_t o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = f32_to_bf16_rne(__builtin_fmaf(acc[i][j][4 * q + e], sc[e], bs[e]));
        uint16_t* orow = g.out + (int64_t)m * g.ldo;
        if (vec_out && nb + 3 < g.N) {
          uint2 v;
          v.x = o[0] | (o[1] << 16);
          v.y = o[2] | (o[3] << 16);
          *reinterpret_cast<uint2*>(orow + nb) = v;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (nb + e < g.N) orow[nb + e] = (uint16_t)o[e];
        }
      }
    }
  }
}

}  // namespace

bool gemm_mfma_supported(const GemmArgs& g) {
  // 16-byte vector loads need aligned rows and K % 16 == 0; 32-bit buffer
  // offsets need a 256-row panel to span less than 2 GiB.
  return ((uintptr_t)g.a % 16 == 0) && ((uintptr_t)g.w % 16 == 0) && (g.lda % 16 == 0) && (g.ldw % 16 == 0) &&
         (g.K % 16 == 0) && (int64_t)BM * g.lda < (1ll << 31) && (int64_t)BN * g.ldw < (1ll << 31);
}

hipError_t launch_gemm_mfma(const GemmArgs& g, bool fp8_accumulate, hipStream_t stream) {
  const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
  const unsigned grid = (unsigned)(tiles_m * tiles_n);
  if (fp8_accumulate)
    gemm_mfma_kernel<false><<<grid, kThreads, 0, stream>>>(g, tiles_m, tiles_n);
  else
    gemm_mfma_kernel<true><<<grid, kThreads, 0, stream>>>(g, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace fp8w8a8
