// Scaled FP8 GEMM on the gfx950 matrix cores for M > 64 (prefill; also 49
// to 64 rows on the widest weights), with the rescale epilogue fused into
// the store.
//
// out[m, n] = bf16( sum_k A[m, k] * W[n, k] * (s_a * s_w[n]) + bias[n] ):
// the W8A8 linear of "Prototype FP8Linear W8A8 runtime quantization"
// (opening post), with the channelwise rescale that "[Kernel] Implement
// fallback for FP8 channelwise using torch._scaled_mm" (description) runs
// as a separate pass after the per-tensor GEMM applied here in the store.
//
// Design for CDNA4:
//   * 256 x 256 output tile, 128 k per step; 4 waves, each owning a
//     128 x 128 quarter as 4 x 4 blocks of 32 x 32 matrix-core products
//     (256 fp32 accumulators per lane).  Where such tiles are too few to
//     occupy the GPU (M of a few hundred to a few thousand rows), the same
//     kernel runs 128 x 128 tiles: 2 x 2 blocks per wave, 64 accumulators,
//     everything below scaled to the tile (template WB, blocks per wave
//     and dimension).
//   * Both operands are K-contiguous ([M, K] and [N, K]), the matrix cores'
//     native operand layout: every lane reads 32 contiguous k-bytes of one
//     row, so no transposition is needed anywhere.
//   * Persistent: one workgroup per compute unit (two with 128 x 128 tiles)
//     walks tiles b, b + grid, ... and the operand pipeline runs across tile
//     boundaries.
//   * Global -> LDS directly (buffer_load ... lds, no staging registers),
//     two stages of 64 KiB (32 KiB with 128 x 128 tiles).  Out-of-range
//     lanes (rows past M or N, k past K) return zeros through the buffer
//     range check, so edge tiles need no branches and k tails add nothing.
//   * One barrier per k step, in its middle.  A step's products are split
//     in two halves of 64 k.  Before the barrier the wave multiplies the
//     first half (whose fragments it read during the previous step) and
//     reads the second half's fragments; after it, it multiplies the second
//     half while it reads the NEXT step's first-half fragments from the
//     other stage and issues the DMA loads of the step after next into the
//     stage it has just finished reading.  So no product ever waits for an
//     LDS read at a step boundary, and the barrier, reached with products
//     still queued in the matrix pipe, costs no idle matrix cycles when the
//     waves arrive together.  The barrier also orders the two stage uses:
//     every wave's second-half reads of this stage and every wave's loads
//     of the other stage are complete at it.
//   * In fp8 mode each step also touches, one step ahead of its DMA loads,
//     this workgroup's share of the lines its XCD's concurrent tiles will
//     read (4-byte DMA loads into a junk LDS area), so the DMA loads find
//     them in L2.
//   * Loads and fragment reads are spread between pairs of products (pinned
//     with scheduling barriers): issued in one burst, a wave's load
//     instructions stall its instruction stream on the texture unit while
//     the matrix pipe idles.
//   * LDS rows are 128 bytes; the 16-byte chunk c of row r is stored at
//     position c ^ (r & 7) ^ ((r >> 3) & 1), so the rows that consecutive
//     lanes read land in different bank groups.
//   * Epilogue through LDS: a tile's last step issues no loads, so the stage
//     it read is free; each wave parks 32 accumulator rows at a time (fp32,
//     straight from the accumulator registers) in the part of that stage its
//     own loads fill, reads them back as 8 consecutive columns per lane,
//     applies s_a * s_w[n] and the bias (staged in LDS by DMA at the tile's
//     first step, double-buffered across tiles), and writes 16-byte bf16
//     chunks; a buffer resource's range check drops rows past M.  Then it
//     issues the deferred loads into that same part (no other wave touches
//     it, so no barrier is needed) and reads the next step's fragments.
//   * Tile order: the hardware deals workgroups round-robin to the 8 XCDs;
//     the tile index is remapped so each XCD owns a contiguous run of tiles,
//     and that run walks groups of 8 tile-rows, so the A and W panels a
//     group touches stay in that XCD's L2.
//   * The accumulation is per tile, in a fixed order: results are
//     deterministic.
//   * Two accumulation modes (template EXACT).  The fp8 instruction
//     (v_mfma_f32_32x32x64_f8f6f4) sums each aligned group of 8 products
//     keeping only 13 bits below the group's largest product (measured on
//     gfx950): twice the throughput, but small products beside large ones
//     are truncated.  EXACT converts each fp8 fragment to bf16 in registers
//     (exact: every e4m3 value is a bf16 value) and runs
//     v_mfma_f32_32x32x16_bf16, whose sums keep fp32-class precision; the
//     LDS tiles, the loads and the HBM traffic are the same in both modes.

#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace fp8w8a8 {

namespace {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

constexpr int BK = 128;
constexpr int kThreads = 256;
constexpr int kGroupM = 8;
// L2 prefetch: two 4-byte-per-lane DMA loads per wave and step, landing in a
// junk LDS area nobody reads (512 bytes per wave)
constexpr int kPrefetchBytes = 4 * 512;

// Tile geometry.  WB = 32 x 32 product blocks per wave in each dimension;
// the 4 waves of a workgroup form a 2 x 2 grid, so a tile is TILE x TILE
// with TILE = 64 WB: 256 (WB = 4), or 128 (WB = 2) for problems whose
// 256 x 256 tiles are too few to occupy the GPU.
template <int WB>
struct Geo {
  static constexpr int TILE = 64 * WB;
  static constexpr int kOperandBytes = TILE * BK;  // per operand per stage (32 KiB at TILE 256)
  static constexpr int kStageBytes = 2 * kOperandBytes;
  // per-tile epilogue parameters: TILE column scales (fp32) and biases (bf16)
  static constexpr int kEpiParamBytes = TILE * 4 + TILE * 2;
  static constexpr int kLdsBytes = 2 * kStageBytes + 2 * kEpiParamBytes + kPrefetchBytes;
  static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
  // 8-row (1 KiB) DMA blocks each wave loads per operand and step
  static constexpr int NB = TILE / 32;
  static constexpr int kStepLoads = 2 * NB;  // DMA instructions per wave and step
};
// vector-memory instructions a wave issues besides the operand loads: the L2
// prefetch after each step's loads (fp8 mode) and the two parameter loads at
// a tile's first step
constexpr int kPrefetchOps = 2;
// how many steps the L2 prefetch runs ahead of the DMA loads
constexpr int kPrefetchAhead = 1;
constexpr int kParamOps = 2;

// XOR swizzle of the 16-byte chunks of a 128-byte LDS row.  The 16 rows a
// half-wave reads at one logical chunk land on 16 distinct (bank-pair,
// chunk) slots, conflict-free whether the LDS serves 8 or 16 lanes of a
// 16-byte read per cycle.
__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }
__device__ __forceinline__ int lds_off(int row, int chunk) { return row * BK + ((chunk ^ swz(row)) << 4); }

__device__ __forceinline__ v8i read_frag(const uint8_t* base, int row, int chunk) {
  const v4i lo = *reinterpret_cast<const v4i*>(base + lds_off(row, chunk));
  const v4i hi = *reinterpret_cast<const v4i*>(base + lds_off(row, chunk + 1));
  v8i f;
  f[0] = lo[0]; f[1] = lo[1]; f[2] = lo[2]; f[3] = lo[3];
  f[4] = hi[0]; f[5] = hi[1]; f[6] = hi[2]; f[7] = hi[3];
  return f;
}

// 4 fp8 codes of format F -> 4 bf16 values of dst starting at element `at`
// (exact).
template <int F>
__device__ __forceinline__ void fp8x4_to_bf16(int w, bf16x8& dst, int at) {
  bf16x2 lo = fp8x2_to_bf16<F, false>(w);
  bf16x2 hi = fp8x2_to_bf16<F, true>(w);
  dst[at] = lo[0]; dst[at + 1] = lo[1]; dst[at + 2] = hi[0]; dst[at + 3] = hi[1];
}

template <int F>
__device__ __forceinline__ bf16x8 slice_bf16(const v8i& f, int t) {
  bf16x8 b;
  fp8x4_to_bf16<F>(f[2 * t], b, 0);
  fp8x4_to_bf16<F>(f[2 * t + 1], b, 4);
  return b;
}

// Where one tile lives: its origin and buffer resources for the two operands
// and the output, each based at the tile's first row.
struct Tile {
  int m0, n0, cols;
  __amdgpu_buffer_rsrc_t ra, rw, ro;
};

template <int TILE>
__device__ __forceinline__ Tile tile_at(const GemmArgs& g, int b, int tiles_m, int tiles_n) {
  constexpr int BM = TILE, BN = TILE;
  const int T = tiles_m * tiles_n;
  if ((T & 7) == 0) b = (b & 7) * (T >> 3) + (b >> 3);
  const int per_group = kGroupM * tiles_n;
  const int first_m = (b / per_group) * kGroupM;
  const int gm = min(tiles_m - first_m, kGroupM);
  Tile t;
  const int tm = first_m + (b % per_group) % gm;
  const int tn = (b % per_group) / gm;
  t.m0 = tm * BM;
  t.n0 = tn * BN;
  const int rows_a = min(BM, g.M - t.m0), rows_w = min(BN, g.N - t.n0);
  t.cols = rows_w;
  // A row r >= rows sits at offset >= rows * ld >= (rows - 1) * ld + K, past
  // the range, so rows beyond M (or N) read as zeros.
  const uint32_t nrec_a = (uint32_t)((int64_t)(rows_a - 1) * g.lda + g.K);
  const uint32_t nrec_w = (uint32_t)((int64_t)(rows_w - 1) * g.ldw + g.K);
  const uint32_t nrec_o = (uint32_t)(((int64_t)(rows_a - 1) * g.ldo + rows_w) * 2);
  t.ra = __builtin_amdgcn_make_buffer_rsrc((void*)(g.a + (int64_t)t.m0 * g.lda), (short)0, (int)nrec_a, kRsrcWord3);
  t.rw = __builtin_amdgcn_make_buffer_rsrc((void*)(g.w + (int64_t)t.n0 * g.ldw), (short)0, (int)nrec_w, kRsrcWord3);
  t.ro = __builtin_amdgcn_make_buffer_rsrc((void*)(g.out + (int64_t)t.m0 * g.ldo + t.n0), (short)0, (int)nrec_o,
                                           kRsrcWord3);
  return t;
}

// VEC: N % 8 == 0, ldo % 8 == 0 and a 16-byte aligned output, so every lane
// writes whole 16-byte chunks (a fixed count of stores per tile).
template <int WB, bool EXACT, bool VEC, int FA, int FW>
__global__ __launch_bounds__(kThreads, 1) void gemm_mfma_kernel(GemmArgs g, int tiles_m, int tiles_n) {
  using G = Geo<WB>;
  constexpr int TILE = G::TILE, HALF = TILE / 2, NB = G::NB;
  constexpr int kOperandBytes = G::kOperandBytes, kStageBytes = G::kStageBytes;
  constexpr int kEpiParamBytes = G::kEpiParamBytes, kStepLoads = G::kStepLoads;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[G::kLdsBytes];
  uint8_t* const params = smem + 2 * kStageBytes;  // two parameter buffers, by tile parity
  uint8_t* const pf_junk = params + 2 * kEpiParamBytes;

  const int T = tiles_m * tiles_n;
  const int KT = (g.K + BK - 1) / BK;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  constexpr int kPf = EXACT ? 0 : kPrefetchOps;

  // ---- loader: buffer_load_dwordx4 ... lds.  Each wave instruction fills
  // one dense 1 KiB LDS block (8 rows x 128 bytes, lane i -> bytes 16i ..
  // 16i+15, the block's base in M0); the XOR swizzle is applied by choosing
  // which global chunk each lane fetches.  Block b of an operand is loaded
  // by wave b / 8.  Lanes whose chunk lies past K, and whole steps past the
  // last tile, load zeros (out-of-range offset).
  uint32_t dvoff_a[NB], dvoff_w[NB];
  const int drow_in_blk = lane >> 3, dphys = lane & 7;
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int row = (wave * NB + i) * 8 + drow_in_blk;
    const int c = dphys ^ swz(row);
    dvoff_a[i] = (uint32_t)(row * g.lda + c * 16);
    dvoff_w[i] = (uint32_t)(row * g.ldw + c * 16);
  }
  // the chunk (hence k offset) a lane fetches depends only on its row within
  // the block and on the block's parity
  const int dchunk_k0 = (dphys ^ drow_in_blk) * 16, dchunk_k1 = (dphys ^ drow_in_blk ^ 1) * 16;

  // The load cursor: the tile and k step the next DMA loads fetch.  It runs
  // two steps ahead of the products, across tile boundaries; past the last
  // tile its loads fetch zeros.
  int lb = blockIdx.x, lkt = 0;
  Tile lt = tile_at<TILE>(g, lb, tiles_m, tiles_n);
  auto advance_load = [&]() {
    if (++lkt == KT) {
      lkt = 0;
      lb += gridDim.x;
      if (lb < T) lt = tile_at<TILE>(g, lb, tiles_m, tiles_n);
    }
  };
  // one block of each operand of the load cursor's step (2 instructions)
  auto dma_part = [&](int stage, int i) {
    const int k0 = lkt * BK;
    const bool kin = lb < T && k0 + ((i & 1) ? dchunk_k1 : dchunk_k0) < g.K;
    uint8_t* As = smem + stage * kStageBytes;
    uint8_t* Ws = As + kOperandBytes;
    const int blk = __builtin_amdgcn_readfirstlane(wave * NB + i);
    const uint32_t oa = kin ? dvoff_a[i] + k0 : kOutOfRange;
    const uint32_t ow = kin ? dvoff_w[i] + k0 : kOutOfRange;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(lt.ra, (__attribute__((address_space(3))) void*)(As + blk * 1024), 16,
                                             (int)oa, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(lt.rw, (__attribute__((address_space(3))) void*)(Ws + blk * 1024), 16,
                                             (int)ow, 0, 0, 0);
  };
  // The prefetch cursor: kPrefetchAhead steps ahead of the load cursor.
  int pb = blockIdx.x, pkt = 0;
  Tile pt = lt;
  auto advance_prefetch = [&]() {
    if (++pkt == KT) {
      pkt = 0;
      pb += gridDim.x;
      if (pb < T) pt = tile_at<TILE>(g, pb, tiles_m, tiles_n);
    }
  };
  // L2 prefetch of the prefetch cursor's step, which then advances.
  // The 32 workgroups an XCD runs at once hold 8 tile-rows x 4 tile-columns
  // (see tile_at), so they share 8 A panels (4 tiles each) and 4 W panels
  // (8 tiles each): this one touches rows 64 (tn % 4) .. + 63 of its A panel
  // and 32 (tm % 8) .. + 31 of its W panel, one line per row, so together
  // they bring each panel's step into the XCD's L2.  The loads land in a
  // junk LDS area (no registers to hold, nothing waits on them); for other
  // tile layouts they merely touch lines of this tile's own panels.
  auto prefetch = [&]() {
    const int tm = pt.m0 / TILE, tn = pt.n0 / TILE;
    const bool valid = pb < T;
    const int s = pkt * BK;
    const uint32_t oa =
        (valid && lane < TILE / 16) ? (uint32_t)(((TILE / 4) * (tn & 3) + (TILE / 16) * wave + lane) * g.lda + s)
                                    : kOutOfRange;
    const uint32_t ow =
        (valid && lane < TILE / 32) ? (uint32_t)(((TILE / 8) * (tm & 7) + (TILE / 32) * wave + lane) * g.ldw + s)
                                    : kOutOfRange;
    uint8_t* J = pf_junk + __builtin_amdgcn_readfirstlane(wave * 512);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(pt.ra, (__attribute__((address_space(3))) void*)J, 4, (int)oa, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(pt.rw, (__attribute__((address_space(3))) void*)(J + 256), 4, (int)ow, 0,
                                             0, 0);
    advance_prefetch();
  };

  const int frow = lane & 31;          // operand row within a 32-row block
  const int fchunk = (lane >> 5) * 2;  // first of the lane's two chunks
  const float sa = *g.s_a;

  // scales and bias through buffer resources: a missing bias is a resource of
  // size 0, whose loads return zeros
  const __amdgpu_buffer_rsrc_t rsw = __builtin_amdgcn_make_buffer_rsrc(
      (void*)g.s_w, (short)0, g.per_channel ? g.N * 4 : 4, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rbias = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(g.bias ? g.bias : reinterpret_cast<const uint16_t*>(g.s_w)), (short)0, g.bias ? g.N * 2 : 0,
      kRsrcWord3);
  // a tile's epilogue parameters, straight into LDS (no registers, so no wait
  // on them lands before the epilogue), exactly kParamOps instructions per
  // wave: wave w fetches the scales of columns 64w .. 64w + 63 and the
  // biases of columns 64w .. 64w + 63 (two per lane for waves 0 and 1, a
  // load of nothing for waves 2 and 3); columns past N read zeros and are
  // never stored.
  auto load_params = [&](const Tile& t, uint8_t* P) {
    float* Psc = reinterpret_cast<float*>(P);
    uint16_t* Pbias = reinterpret_cast<uint16_t*>(P + TILE * 4);
    // waves past the tile's columns (TILE 128: waves 2 and 3 for the scales,
    // 1 to 3 for the biases) load nothing into the junk area
    const bool sc_wave = TILE >= 4 * 64 || wave < TILE / 64;
    const int nc = t.n0 + wave * 64 + lane;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rsw,
        (__attribute__((address_space(3))) void*)(sc_wave ? Psc + __builtin_amdgcn_readfirstlane(wave * 64)
                                                          : reinterpret_cast<float*>(pf_junk)),
        4, (int)(!sc_wave ? kOutOfRange : g.per_channel ? (nc < g.N ? (uint32_t)nc * 4 : kOutOfRange) : 0u), 0, 0, 0);
    // VEC: N % 8 == 0, so no dword of two biases straddles the end
    const int nb2 = t.n0 + (wave & 1) * 128 + 2 * lane;
    const bool bias_ok = VEC && wave < TILE / 128 && nb2 < g.N;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rbias,
        (__attribute__((address_space(3))) void*)(wave < TILE / 128
                                                      ? Pbias + __builtin_amdgcn_readfirstlane(wave * 128)
                                                      : reinterpret_cast<uint16_t*>(pf_junk)),
        4, (int)(bias_ok ? (uint32_t)nb2 * 2 : kOutOfRange), 0, 0, 0);
  };

  // ---- prologue: the first two steps' loads, then the first step's
  // first-half fragments
#pragma unroll
  for (int i = 0; i < NB; ++i) dma_part(0, i);
  advance_load();
#pragma unroll
  for (int i = 0; i < NB; ++i) dma_part(1, i);
  advance_load();
  advance_prefetch();
  advance_prefetch();
  if constexpr (!EXACT) {
#pragma unroll
    for (int d = 0; d < kPrefetchAhead; ++d) prefetch();
  }
  __builtin_amdgcn_s_waitcnt(wait_vmcnt(kStepLoads + kPf * kPrefetchAhead));
  __builtin_amdgcn_s_barrier();
  v8i wf0[WB], af0[WB], wf1[WB], af1[WB];
#pragma unroll
  for (int i = 0; i < WB; ++i) wf0[i] = read_frag(smem + kOperandBytes, wn * HALF + i * 32 + frow, fchunk);
#pragma unroll
  for (int j = 0; j < WB; ++j) af0[j] = read_frag(smem, wm * HALF + j * 32 + frow, fchunk);

  int step = 0;   // steps done over all tiles: stage parity
  int tcount = 0;  // tiles done: parameter-buffer parity
  v16f acc[WB][WB];
  // product pairs per half step (fp8 mode), and per pair: fragment reads and
  // DMA parts (one of each at WB = 4)
  constexpr int NP = WB * WB / 2, RPP = 2 * WB / NP, DPP = NB / NP;
  // exact mode: DMA parts per 16-deep slice
  constexpr int DPT = NB / 4;
  // One k step (see the design notes above).  FIRST: the tile's first step
  // (its parameter loads).  LAST: the tile's last step, whose second half
  // issues no loads and reads no fragments: its stage becomes the
  // epilogue's staging area, and the loads of the step after next and the
  // next step's fragment reads follow the epilogue.
  auto do_step = [&](auto first_c, auto last_c, const Tile& cur, uint8_t* P) {
    constexpr bool FIRST = decltype(first_c)::value;
    constexpr bool LAST = decltype(last_c)::value;
    const uint8_t* As = smem + (step & 1) * kStageBytes;
    const uint8_t* Ws = As + kOperandBytes;
    const uint8_t* An = smem + ((step + 1) & 1) * kStageBytes;
    const uint8_t* Wn = An + kOperandBytes;
    // this step's first-half fragments (read during the previous step) are in
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    if constexpr (FIRST) load_params(cur, P);
    __builtin_amdgcn_sched_barrier(0);
    // ---- first half: its products, with the second half's fragment reads
    if constexpr (!EXACT) {
#pragma unroll
      for (int p = 0; p < NP; ++p) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int i = (2 * p + q) / WB, j = (2 * p + q) % WB;
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wf0[i], af0[j], acc[i][j], FW, FA, 0, 0, 0,
                                                                       0);
        }
#pragma unroll
        for (int r = p * RPP; r < (p + 1) * RPP; ++r) {
          if (r < WB) wf1[r] = read_frag(Ws, wn * HALF + r * 32 + frow, 4 + fchunk);
          else af1[r - WB] = read_frag(As, wm * HALF + (r - WB) * 32 + frow, 4 + fchunk);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        bf16x8 wb[WB], ab[WB];
#pragma unroll
        for (int i = 0; i < WB; ++i) wb[i] = slice_bf16<FW>(wf0[i], t);
#pragma unroll
        for (int j = 0; j < WB; ++j) ab[j] = slice_bf16<FA>(af0[j], t);
#pragma unroll
        for (int i = 0; i < WB; ++i)
#pragma unroll
          for (int j = 0; j < WB; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wb[i], ab[j], acc[i][j], 0, 0, 0);
        if (t < WB) {
          wf1[t] = read_frag(Ws, wn * HALF + t * 32 + frow, 4 + fchunk);
          af1[t] = read_frag(As, wm * HALF + t * 32 + frow, 4 + fchunk);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // ---- the step's barrier.  Outstanding vector-memory operations of this
    // wave, oldest first: the next step's loads (issued during the previous
    // step, or after the previous tile's epilogue), their L2 prefetch, and
    // at a tile's first step its parameter loads; in-order completion lets
    // the wait leave everything after the loads in flight.  The second-half
    // reads of this stage are done too, so after the barrier every wave may
    // overwrite it.
    if constexpr (!FIRST)
      __builtin_amdgcn_s_waitcnt(wait_vmcnt(kPf) & kWaitLgkm0);
    else
      __builtin_amdgcn_s_waitcnt(wait_vmcnt(kPf + kParamOps) & kWaitLgkm0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    // ---- second half: its products, with the loads of the step after next
    // into this stage and (but in a tile's last step) the next step's
    // first-half fragment reads
    if constexpr (!EXACT) {
#pragma unroll
      for (int p = 0; p < NP; ++p) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int i = (2 * p + q) / WB, j = (2 * p + q) % WB;
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wf1[i], af1[j], acc[i][j], FW, FA, 0, 0, 0,
                                                                       0);
        }
        if constexpr (!LAST) {
#pragma unroll
          for (int d = p * DPP; d < (p + 1) * DPP; ++d) dma_part(step & 1, d);
          if (p == NP - 1) {
            advance_load();
            prefetch();
          }
#pragma unroll
          for (int r = p * RPP; r < (p + 1) * RPP; ++r) {
            if (r < WB) wf0[r] = read_frag(Wn, wn * HALF + r * 32 + frow, fchunk);
            else af0[r - WB] = read_frag(An, wm * HALF + (r - WB) * 32 + frow, fchunk);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        bf16x8 wb[WB], ab[WB];
#pragma unroll
        for (int i = 0; i < WB; ++i) wb[i] = slice_bf16<FW>(wf1[i], t);
#pragma unroll
        for (int j = 0; j < WB; ++j) ab[j] = slice_bf16<FA>(af1[j], t);
#pragma unroll
        for (int i = 0; i < WB; ++i)
#pragma unroll
          for (int j = 0; j < WB; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wb[i], ab[j], acc[i][j], 0, 0, 0);
        if constexpr (!LAST) {
#pragma unroll
          for (int d = t * DPT; d < (t + 1) * DPT; ++d) dma_part(step & 1, d);
          if (t == 3) advance_load();
          if (t < WB) {
            wf0[t] = read_frag(Wn, wn * HALF + t * 32 + frow, fchunk);
            af0[t] = read_frag(An, wm * HALF + t * 32 + frow, fchunk);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    ++step;
  };
  using True = std::integral_constant<bool, true>;
  using False = std::integral_constant<bool, false>;

  for (int b = blockIdx.x; b < T; b += gridDim.x, ++tcount) {
    const Tile cur = tile_at<TILE>(g, b, tiles_m, tiles_n);
    uint8_t* const P = params + (tcount & 1) * kEpiParamBytes;
#pragma unroll
    for (int i = 0; i < WB; ++i)
#pragma unroll
      for (int j = 0; j < WB; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
    if (KT == 1) {
      do_step(True(), True(), cur, P);
    } else {
      do_step(True(), False(), cur, P);
      for (int kt = 1; kt < KT - 1; ++kt) do_step(False(), False(), cur, P);
      do_step(False(), True(), cur, P);
    }

    // ---- epilogue.  acc[i][j] = D[n][m] for the 32x32 block (i: n, j: m):
    // lane holds m = lane % 32 and, in registers 4q..4q+3, the four
    // consecutive columns n = 8q + 4 * (lane / 32) + 0..3.  Each round parks
    // the 32 rows of block-row j (fp32, HALF columns: LDS rows of 4 HALF
    // bytes, 16-byte chunk c of row r at c ^ r over the row's chunks) in the
    // last step's stage -- rows 0..15 in the NB KiB of its A part and rows
    // 16..31 in the NB KiB of its W part that this wave's own loads fill, so
    // no other wave touches them -- and reads them back as 8 consecutive
    // columns per lane.
    if (KT == 1) {
      // a one-step tile: its parameter loads were issued this very step
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      __builtin_amdgcn_s_barrier();
    }
    const int lstage = (step - 1) & 1;  // the stage the tile's last step read
    uint8_t* const Spark = smem + lstage * kStageBytes;
    float* const E0 = reinterpret_cast<float*>(Spark + wave * NB * 1024);                  // rows 0..15
    float* const E1 = reinterpret_cast<float*>(Spark + kOperandBytes + wave * NB * 1024);  // rows 16..31
    // a parked row: HALF floats, CPR groups of 8 columns, 2 CPR 16-byte chunks
    constexpr int CPR = HALF / 8, CMASK = 2 * CPR - 1, RPS = 64 / CPR, CPR_LOG2 = WB == 4 ? 4 : 3;
    static_assert((1 << CPR_LOG2) == CPR, "column groups per parked row");
    // The lane index, made opaque to the compiler here: the epilogue's
    // per-lane LDS addresses and store offsets are loop-invariant, and
    // hoisted out of the tile loop they would occupy (and spill) some sixty
    // registers for the whole kernel.
    int elane = lane;
    asm volatile("" : "+v"(elane));
    // read-back role: columns 8 ec .. + 7 of rows er + RPS s
    const int ec = elane & (CPR - 1), er = (elane >> CPR_LOG2) & (RPS - 1);
    const int ecol = wn * HALF + ec * 8;        // within the tile
    const bool col_ok = cur.n0 + ecol + 8 <= g.N;
    float sc[8], bs[8];
    {
      const float* Psc = reinterpret_cast<const float*>(P);
      const uint16_t* Pbias = reinterpret_cast<const uint16_t*>(P + TILE * 4);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        sc[e] = sa * Psc[ecol + e];
        if constexpr (VEC)
          bs[e] = bf16_to_f32(Pbias[ecol + e]);
        else
          bs[e] = g.bias ? bf16_to_f32(g.bias[min(cur.n0 + ecol + e, g.N - 1)]) : 0.0f;
      }
    }
#pragma unroll
    for (int j = 0; j < WB; ++j) {
      {
        const int r = elane & 31;
        float* const E = r < 16 ? E0 : E1;
        const int rl = r & 15;
#pragma unroll
        for (int i = 0; i < WB; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int c = i * 8 + 2 * q + ((elane >> 5) & 1);
            v4f v;
            v[0] = acc[i][j][4 * q]; v[1] = acc[i][j][4 * q + 1];
            v[2] = acc[i][j][4 * q + 2]; v[3] = acc[i][j][4 * q + 3];
            *reinterpret_cast<v4f*>(E + rl * HALF + ((c ^ (r & CMASK)) << 2)) = v;
          }
      }
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int s8 = 0; s8 < 32 / RPS; ++s8) {
        const int rr = s8 * RPS + er;
        const float* E = rr < 16 ? E0 : E1;
        const int rl = rr & 15;
        const v4f lo = *reinterpret_cast<const v4f*>(E + rl * HALF + (((2 * ec) ^ (rr & CMASK)) << 2));
        const v4f hi = *reinterpret_cast<const v4f*>(E + rl * HALF + (((2 * ec + 1) ^ (rr & CMASK)) << 2));
        // columns 8 ec + 0..7 as bf16 pairs (one conversion instruction each)
        v4u packed;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          packed[e] = pack_bf16x2_rne(__builtin_fmaf(lo[2 * e], sc[2 * e], bs[2 * e]),
                                      __builtin_fmaf(lo[2 * e + 1], sc[2 * e + 1], bs[2 * e + 1]));
          packed[e + 2] = pack_bf16x2_rne(__builtin_fmaf(hi[2 * e], sc[2 * e + 4], bs[2 * e + 4]),
                                          __builtin_fmaf(hi[2 * e + 1], sc[2 * e + 5], bs[2 * e + 5]));
        }
        const int row = wm * HALF + j * 32 + rr;  // within the tile
        if constexpr (VEC) {
          const uint32_t off = col_ok ? (uint32_t)((row * g.ldo + ecol) * 2) : kOutOfRange;
          __builtin_amdgcn_raw_buffer_store_b128(packed, cur.ro, (int)off, 0, 0);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t off = ecol + e < cur.cols ? (uint32_t)((row * g.ldo + ecol + e) * 2) : kOutOfRange;
            __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(packed[e >> 1] >> (16 * (e & 1))), cur.ro, (int)off, 0,
                                                  0);
          }
        }
      }
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      __builtin_amdgcn_wave_barrier();  // the next round rewrites E
    }
    // the deferred loads of the step after next go into this wave's own part
    // of the stage it has just finished reading; then the next step's
    // first-half fragments (their loads landed before the last barrier)
#pragma unroll
    for (int i = 0; i < NB; ++i) dma_part(lstage, i);
    advance_load();
    if constexpr (!EXACT) prefetch();
    {
      const uint8_t* An = smem + (step & 1) * kStageBytes;
      const uint8_t* Wn = An + kOperandBytes;
#pragma unroll
      for (int i = 0; i < WB; ++i) wf0[i] = read_frag(Wn, wn * HALF + i * 32 + frow, fchunk);
#pragma unroll
      for (int j = 0; j < WB; ++j) af0[j] = read_frag(An, wm * HALF + j * 32 + frow, fchunk);
    }
  }
  // loads past the last tile still write (zeros) into LDS: let them land
  // before the workgroup's LDS is released
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
}

int cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64 && cached[dev] > 0) return cached[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  if (dev < 64) cached[dev] = n;
  return n;
}

}  // namespace

bool gemm_mfma_supported(const GemmArgs& g) {
  // 16-byte vector loads need aligned rows and K % 16 == 0; 32-bit buffer
  // offsets need a panel of the larger tile (256 rows of the operands and
  // the output) to span less than 2 GiB.
  constexpr int64_t kPanelRows = Geo<4>::TILE;
  return ((uintptr_t)g.a % 16 == 0) && ((uintptr_t)g.w % 16 == 0) && (g.lda % 16 == 0) && (g.ldw % 16 == 0) &&
         (g.K % 16 == 0) && kPanelRows * g.lda < (1ll << 31) && kPanelRows * g.ldw < (1ll << 31) &&
         kPanelRows * g.ldo * 2 < (1ll << 31) && ((uintptr_t)g.out % 2 == 0) && g.N < (1 << 29);
}

template <int WB, int FA, int FW>
hipError_t launch_mfma_tiles(const GemmArgs& g, bool fp8_accumulate, hipStream_t stream) {
  constexpr int TILE = Geo<WB>::TILE;
  // in 64 bits: M may come within a tile of 2^31
  const int tiles_m = (int)(((int64_t)g.M + TILE - 1) / TILE), tiles_n = (int)(((int64_t)g.N + TILE - 1) / TILE);
  const int T = tiles_m * tiles_n;
  // 128 x 128 tiles: two workgroups fit a CU (128 VGPRs and 64 accumulation
  // registers per lane of its 512, and 68 KiB of LDS, each; asking the
  // compiler for two per CU moved the accumulators into VGPRs, within 2-4%
  // of the same speed), and where the tiles outnumber the CUs
  // two resident workgroups overlap one's loads with the other's products:
  // 12-19% faster than one per CU (M = 2048 on N = 4096: 74.6 -> 64.8 us;
  // M = 320 on N = 14336: 72.6 -> 58.7 us), no change with fewer tiles.
  const unsigned grid = (unsigned)min(T, (WB == 2 ? 2 : 1) * cu_count());
  const bool vec = (g.N % 8 == 0) && (g.ldo % 8 == 0) && ((uintptr_t)g.out % 16 == 0);
  if (fp8_accumulate) {
    if (vec)
      gemm_mfma_kernel<WB, false, true, FA, FW><<<grid, kThreads, 0, stream>>>(g, tiles_m, tiles_n);
    else
      gemm_mfma_kernel<WB, false, false, FA, FW><<<grid, kThreads, 0, stream>>>(g, tiles_m, tiles_n);
  } else {
    if (vec)
      gemm_mfma_kernel<WB, true, true, FA, FW><<<grid, kThreads, 0, stream>>>(g, tiles_m, tiles_n);
    else
      gemm_mfma_kernel<WB, true, false, FA, FW><<<grid, kThreads, 0, stream>>>(g, tiles_m, tiles_n);
  }
  return hipGetLastError();
}

// Tile size.  Each CU runs one 256 x 256 tile at a time, or two 128 x 128
// tiles (see launch_mfma_tiles).  A 128 x 128 tile (a quarter of the work,
// four times the DMA loads per product) took 0.45 of a 256 x 256 tile's
// time with fp32-class sums and 0.58 with fp8 sums (K = 4096), and a
// partial last round of tiles cost about its share (the part is
// power-limited: CUs left idle let the others clock up).  So 128 x 128 tiles
// run where max(1, tiles / CUs) tile times is the smaller estimate.
// Measured: M = 320 to 1024 on N = 4096 went from 80-82 to 36-42 us with
// fp32-class sums and from 47-52 to 28-30 us with fp8 sums; M = 2048 on
// N = 6144 stays on 256 x 256 (98 against 111 us).
template <int FA, int FW>
hipError_t launch_mfma(const GemmArgs& g, bool fp8_accumulate, hipStream_t stream) {
  const int64_t cus = cu_count();
  const int64_t M = g.M, N = g.N;
  const int64_t tiles256 = ((M + 255) / 256) * ((N + 255) / 256);
  const int64_t tiles128 = ((M + 127) / 128) * ((N + 127) / 128);
  const bool small = std::max(cus, tiles128) * (fp8_accumulate ? 58 : 45) < std::max(cus, tiles256) * 100;
  if (small) return launch_mfma_tiles<2, FA, FW>(g, fp8_accumulate, stream);
  return launch_mfma_tiles<4, FA, FW>(g, fp8_accumulate, stream);
}

hipError_t launch_gemm_mfma(const GemmArgs& g, bool fp8_accumulate, hipStream_t stream) {
  if (g.fmt_a == kE5M2)
    return g.fmt_w == kE5M2 ? launch_mfma<kE5M2, kE5M2>(g, fp8_accumulate, stream)
                            : launch_mfma<kE5M2, kE4M3>(g, fp8_accumulate, stream);
  return g.fmt_w == kE5M2 ? launch_mfma<kE4M3, kE5M2>(g, fp8_accumulate, stream)
                          : launch_mfma<kE4M3, kE4M3>(g, fp8_accumulate, stream);
}

}  // namespace fp8w8a8
