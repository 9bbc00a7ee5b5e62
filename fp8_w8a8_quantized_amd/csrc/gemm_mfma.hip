// Scaled FP8 GEMM on the gfx950 matrix cores for M > 64 (prefill), with the
// rescale epilogue fused into the store.
//
// out[m, n] = bf16( sum_k A[m, k] * W[n, k] * (s_a * s_w[n]) + bias[n] ):
// the W8A8 linear of "Prototype FP8Linear W8A8 runtime quantization"
// (opening post), with the channelwise rescale that "[Kernel] Implement
// fallback for FP8 channelwise using torch._scaled_mm" (description) runs
// as a separate pass after the per-tensor GEMM applied here in the store.
//
// Design for CDNA4:
//   * 256 x 256 output tile, 128 k per step; 4 waves, each owning a
//     128 x 128 quarter as 4 x 4 blocks of v_mfma_f32_32x32x64_f8f6f4
//     (256 fp32 accumulators per lane).
//   * Both operands are K-contiguous ([M, K] and [N, K]), the matrix cores'
//     native operand layout: every lane reads 32 contiguous k-bytes of one
//     row, so no transposition is needed anywhere.
//   * Persistent: one workgroup per compute unit walks tiles b, b + grid, ...
//     The operand pipeline runs across tile boundaries (the last k step of a
//     tile loads the next tile's first step), and the epilogue's stores
//     drain while the next tile's first step computes.
//   * Global -> LDS directly (buffer_load ... lds, no staging registers),
//     double-buffered (2 x 64 KiB).  Out-of-range lanes (rows past M or N,
//     k past K) return zeros through the buffer range check, so edge tiles
//     need no branches and k tails add nothing.
//   * In fp8 mode each step also touches, two steps ahead, this
//     workgroup's share of the lines its XCD's concurrent tiles will read
//     (4-byte DMA loads into a junk LDS area), so the step's own loads find
//     them in L2 (measured: +5%; the bf16 mode, twice as long per step, does
//     not gain from it).
//   * Issue order within a k step (pinned with scheduling barriers): the
//     first half's fragments, then the first half's 16 products with one
//     block of the next step's loads and two of the second half's fragment
//     reads after each pair, then the second half's products.  Issued in one
//     burst, the 16 load instructions of a wave stall its instruction stream
//     on the texture unit while the matrix pipe idles (measured: ~30% of
//     the step even with every load hitting L2).
//   * LDS rows are 128 bytes; the 16-byte chunk c of row r is stored at
//     position c ^ (r & 7) ^ ((r >> 3) & 1), so the rows that consecutive
//     lanes read land in different bank groups.
//   * Epilogue through LDS: each wave parks 32 accumulator rows at a time
//     (fp32) in the stage buffer the tile's last step used, reads them back
//     as 8 consecutive columns per lane, applies s_a * s_w[n] and the bias,
//     and writes 16-byte bf16 chunks, a wave instruction covering four
//     256-byte row segments.  The stores go through a buffer resource, whose
//     range check drops rows past M.
//   * Tile order: the hardware deals workgroups round-robin to the 8 XCDs;
//     the tile index is remapped so each XCD owns a contiguous run of tiles,
//     and that run walks groups of 8 tile-rows, so the A and W panels a
//     group touches stay in that XCD's L2.
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

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

constexpr int BM = 256, BN = 256, BK = 128;
constexpr int kThreads = 256;
constexpr int kOperandBytes = BM * BK;  // 32 KiB per operand per stage
constexpr int kStageBytes = 2 * kOperandBytes;
constexpr int kGroupM = 8;
constexpr int kEpiParamBytes = BN * 4 + BN * 2;
// L2 prefetch: two 4-byte-per-lane DMA loads per wave and step, landing in a
// junk LDS area nobody reads (512 bytes per wave)
constexpr int kPrefetchBytes = 4 * 512;
constexpr int kPrefetchOps = 2;
constexpr int kPrefetchDist = 2;
// Epilogue: 32 rows per round, 4 rounds, 8 store instructions per round.
constexpr int kEpiStores = 32;
// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] in bits 3:0, vmcnt[5:4] in
// bits 15:14, expcnt in 6:4, lgkmcnt in 11:8; fields at their maximum do not
// wait).  vmcnt(32) lets the previous tile's 32 epilogue stores, issued after
// the loads being waited for, stay in flight.
// In fp8 mode every step ends with kPrefetchOps prefetch loads, so a step's
// wait leaves them (and after a tile, the epilogue stores issued later) in
// flight.
constexpr int wait_step(bool prefetching) { return wait_vmcnt(prefetching ? kPrefetchOps : 0); }
constexpr int wait_epi(bool prefetching) { return wait_vmcnt(kEpiStores + (prefetching ? kPrefetchOps : 0)); }

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

__device__ __forceinline__ Tile tile_at(const GemmArgs& g, int b, int tiles_m, int tiles_n) {
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
template <bool EXACT, bool VEC, int FA, int FW>
__global__ __launch_bounds__(kThreads, 1) void gemm_mfma_kernel(GemmArgs g, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * kStageBytes + kEpiParamBytes + kPrefetchBytes];
  // the tile's 256 column scales (fp32) and biases (bf16), loaded by DMA
  float* Psc = reinterpret_cast<float*>(smem + 2 * kStageBytes);
  uint16_t* Pbias = reinterpret_cast<uint16_t*>(smem + 2 * kStageBytes + BN * 4);

  const int T = tiles_m * tiles_n;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- loader: buffer_load_dwordx4 ... lds.  Each wave instruction fills
  // one dense 1 KiB LDS block (8 rows x 128 bytes, lane i -> bytes 16i ..
  // 16i+15, the block's base in M0); the XOR swizzle is applied by choosing
  // which global chunk each lane fetches.  Block b of an operand is loaded
  // by wave b / 8.  Lanes whose chunk lies past K, and whole steps past the
  // last tile, load zeros (out-of-range offset).
  uint32_t dvoff_a[8], dvoff_w[8];
  const int drow_in_blk = lane >> 3, dphys = lane & 7;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = (wave * 8 + i) * 8 + drow_in_blk;
    const int c = dphys ^ swz(row);
    dvoff_a[i] = (uint32_t)(row * g.lda + c * 16);
    dvoff_w[i] = (uint32_t)(row * g.ldw + c * 16);
  }
  // the chunk (hence k offset) a lane fetches depends only on its row within
  // the block and on the block's parity
  const int dchunk_k0 = (dphys ^ drow_in_blk) * 16, dchunk_k1 = (dphys ^ drow_in_blk ^ 1) * 16;
  // one block of each operand (2 instructions); dma() issues all 8 blocks
  auto dma_part = [&](int stage, const Tile& t, int k0, bool step_valid, int i) {
    const bool kin = step_valid && k0 + ((i & 1) ? dchunk_k1 : dchunk_k0) < g.K;
    uint8_t* As = smem + stage * kStageBytes;
    uint8_t* Ws = As + kOperandBytes;
    const int blk = __builtin_amdgcn_readfirstlane(wave * 8 + i);
    const uint32_t oa = kin ? dvoff_a[i] + k0 : kOutOfRange;
    const uint32_t ow = kin ? dvoff_w[i] + k0 : kOutOfRange;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(t.ra, (__attribute__((address_space(3))) void*)(As + blk * 1024), 16,
                                             (int)oa, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(t.rw, (__attribute__((address_space(3))) void*)(Ws + blk * 1024), 16,
                                             (int)ow, 0, 0, 0);
  };
  auto dma = [&](int stage, const Tile& t, int k0, bool step_valid) {
#pragma unroll
    for (int i = 0; i < 8; ++i) dma_part(stage, t, k0, step_valid, i);
  };

  const int KT = (g.K + BK - 1) / BK;
  // L2 prefetch of step s of tile t, kPrefetchDist steps ahead of the step it
  // feeds.  The 32 workgroups an XCD runs at once hold 8 tile-rows x 4
  // tile-columns (see tile_at), so they share 8 A panels (4 tiles each) and
  // 4 W panels (8 tiles each): this one touches rows 64 (tn % 4) .. + 63 of
  // its A panel and 32 (tm % 8) .. + 31 of its W panel, one line per row,
  // so together they bring each panel's next-but-one step into the XCD's
  // L2 while the current step computes.  The loads land in a junk LDS area
  // (no registers to hold, nothing waits on them); for other tile layouts
  // they merely touch lines of this tile's own panels.
  uint8_t* const pf_junk = smem + 2 * kStageBytes + kEpiParamBytes;
  auto prefetch = [&](const Tile& t, int s, bool valid) {
    const int tm = t.m0 / BM, tn = t.n0 / BN;
    const uint32_t oa =
        (valid && lane < 16) ? (uint32_t)((64 * (tn & 3) + 16 * wave + lane) * g.lda + s * BK) : kOutOfRange;
    const uint32_t ow =
        (valid && lane < 8) ? (uint32_t)((32 * (tm & 7) + 8 * wave + lane) * g.ldw + s * BK) : kOutOfRange;
    uint8_t* J = pf_junk + __builtin_amdgcn_readfirstlane(wave * 512);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(t.ra, (__attribute__((address_space(3))) void*)J, 4, (int)oa, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(t.rw, (__attribute__((address_space(3))) void*)(J + 256), 4, (int)ow, 0,
                                             0, 0);
  };
  const int frow = lane & 31;          // operand row within a 32-row block
  const int fchunk = (lane >> 5) * 2;  // first of the lane's two chunks
  const float sa = *g.s_a;
  // epilogue lane roles: 8 consecutive columns (chunk ec) of rows er + 4s
  const int ec = lane & 15, er = lane >> 4;

  // scales and bias through buffer resources: a missing bias is a resource of
  // size 0, whose loads return zeros
  const __amdgpu_buffer_rsrc_t rsw = __builtin_amdgcn_make_buffer_rsrc(
      (void*)g.s_w, (short)0, g.per_channel ? g.N * 4 : 4, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rbias = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(g.bias ? g.bias : reinterpret_cast<const uint16_t*>(g.s_w)), (short)0, g.bias ? g.N * 2 : 0,
      kRsrcWord3);

  int b = blockIdx.x;
  Tile cur = tile_at(g, b, tiles_m, tiles_n);
  dma(0, cur, 0, true);
  if constexpr (!EXACT) prefetch(cur, 1, KT > 1);
  int step = 0;  // steps issued so far over all tiles: stage parity
  bool first = true;
  for (; b < T; b += gridDim.x) {
    const bool has_next = b + (int)gridDim.x < T;
    const Tile nxt = has_next ? tile_at(g, b + gridDim.x, tiles_m, tiles_n) : cur;

    const int ecol = wn * 128 + ec * 8;  // this lane's 8 output columns, within the tile
    const bool col_ok = ecol + 8 <= cur.cols;

    v16f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    int kt = 0;
    do {  // KT >= 1
      // this wave's loads for this step landed (the previous tile's epilogue
      // stores, issued after them, may still be in flight) ...
      if (VEC && kt == 0 && !first)
        __builtin_amdgcn_s_waitcnt(wait_epi(!EXACT));
      else
        __builtin_amdgcn_s_waitcnt(wait_step(!EXACT));
      __builtin_amdgcn_s_barrier();  // ... and every other wave's
      if (kt == 0) {
        // the epilogue's column scales and biases, straight into LDS (no
        // registers, so no wait on them lands before the epilogue): wave w
        // fetches the scales of columns 64w .. 64w + 63, waves 0 and 1 the
        // biases of 128 columns each, two per lane (columns past N: zeros,
        // never stored)
        const int nc = cur.n0 + wave * 64 + lane;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rsw, (__attribute__((address_space(3))) void*)(Psc + __builtin_amdgcn_readfirstlane(wave * 64)), 4,
            (int)(g.per_channel ? (nc < g.N ? (uint32_t)nc * 4 : kOutOfRange) : 0u), 0, 0, 0);
        if (VEC && wave < 2) {  // N % 8 == 0: no dword straddles the end
          const int nb2 = cur.n0 + wave * 128 + 2 * lane;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              rbias, (__attribute__((address_space(3))) void*)(Pbias + __builtin_amdgcn_readfirstlane(wave * 128)),
              4, (int)(nb2 < g.N ? (uint32_t)nb2 * 2 : kOutOfRange), 0, 0, 0);
        }
      }
      const uint8_t* As = smem + (step & 1) * kStageBytes;
      const uint8_t* Ws = As + kOperandBytes;
      // next step's loads into the idle buffer: this tile's next step, or the
      // next tile's first step (zeros after the last tile)
      const bool last_step = kt + 1 >= KT;
      Tile tgt;
      tgt.ra = last_step ? nxt.ra : cur.ra;
      tgt.rw = last_step ? nxt.rw : cur.rw;
      const int k_next = last_step ? 0 : (kt + 1) * BK;
      const bool v_next = last_step ? has_next : true;
      const int nstage = (step + 1) & 1;
      // order: the first half's fragments; then the first half's 16 products,
      // each pair followed by one block of next-step loads and two of the
      // second half's fragment reads; then the second half's products
      v8i wf[2][4], af[2][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) wf[0][i] = read_frag(Ws, wn * 128 + i * 32 + frow, fchunk);
#pragma unroll
      for (int j = 0; j < 4; ++j) af[0][j] = read_frag(As, wm * 128 + j * 32 + frow, fchunk);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (!EXACT) {
#pragma unroll
        for (int p = 0; p < 8; ++p) {
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int i = (2 * p + q) >> 2, j = (2 * p + q) & 3;
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wf[0][i], af[0][j], acc[i][j], FW, FA,
                                                                         0, 0, 0, 0);
          }
          dma_part(nstage, tgt, k_next, v_next, p);
          if (p == 7) prefetch(cur, kt + kPrefetchDist, kt + kPrefetchDist < KT);
          if (p < 4) wf[1][p] = read_frag(Ws, wn * 128 + p * 32 + frow, 4 + fchunk);
          else af[1][p - 4] = read_frag(As, wm * 128 + (p - 4) * 32 + frow, 4 + fchunk);
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wf[1][i], af[1][j], acc[i][j], FW, FA,
                                                                         0, 0, 0, 0);
      } else {
        // the lane's 32 k-values in four slices of 8 (same slicing for
        // both operands), one bf16 32x32x16 product per slice; two blocks of
        // loads and two fragment reads after each slice of the first half
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            bf16x8 wb[4], ab[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) wb[i] = slice_bf16<FW>(wf[ks][i], t);
#pragma unroll
            for (int j = 0; j < 4; ++j) ab[j] = slice_bf16<FA>(af[ks][j], t);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
              for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wb[i], ab[j], acc[i][j], 0, 0, 0);
            if (ks == 0) {
              dma_part(nstage, tgt, k_next, v_next, 2 * t);
              dma_part(nstage, tgt, k_next, v_next, 2 * t + 1);
              wf[1][t] = read_frag(Ws, wn * 128 + t * 32 + frow, 4 + fchunk);
              af[1][t] = read_frag(As, wm * 128 + t * 32 + frow, 4 + fchunk);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
        }
      }
      ++step;
    } while (++kt < KT);

    // ---- epilogue.  acc[i][j] = D[n][m] for the 32x32 block (i: n, j: m):
    // lane holds m = lane % 32 and, in registers 4q..4q+3, the four
    // consecutive columns n = 8q + 4 * (lane / 32) + 0..3.  Each round parks
    // the 32 rows of block-row j (fp32, 512-byte LDS rows, 16-byte chunk c of
    // row r at c ^ (r & 31)) in this wave's 16 KiB of the stage buffer the
    // last step read, then reads them back as 8 columns per lane.
    // every wave is done reading that buffer, and (for a single-step tile,
    // whose scales no later step waited for) the scales have landed
    if (KT == 1) __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __builtin_amdgcn_s_barrier();
    float sc[8], bs[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sc[e] = sa * Psc[ecol + e];
      if constexpr (VEC)
        bs[e] = bf16_to_f32(Pbias[ecol + e]);
      else
        bs[e] = g.bias ? bf16_to_f32(g.bias[min(cur.n0 + ecol + e, g.N - 1)]) : 0.0f;
    }
    float* E = reinterpret_cast<float*>(smem + ((step - 1) & 1) * kStageBytes + wave * 16384);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = lane & 31;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = i * 8 + 2 * q + (lane >> 5);
          v4f v;
          v[0] = acc[i][j][4 * q]; v[1] = acc[i][j][4 * q + 1];
          v[2] = acc[i][j][4 * q + 2]; v[3] = acc[i][j][4 * q + 3];
          *reinterpret_cast<v4f*>(E + r * 128 + ((c ^ r) << 2)) = v;
        }
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int rr = s * 4 + er;
        const v4f lo = *reinterpret_cast<const v4f*>(E + rr * 128 + (((2 * ec) ^ rr) << 2));
        const v4f hi = *reinterpret_cast<const v4f*>(E + rr * 128 + (((2 * ec + 1) ^ rr) << 2));
        uint32_t o[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          o[e] = f32_to_bf16_rne(__builtin_fmaf(lo[e], sc[e], bs[e]));
          o[e + 4] = f32_to_bf16_rne(__builtin_fmaf(hi[e], sc[e + 4], bs[e + 4]));
        }
        const int row = wm * 128 + j * 32 + rr;  // within the tile
        if constexpr (VEC) {
          v4u packed;
          packed[0] = o[0] | (o[1] << 16); packed[1] = o[2] | (o[3] << 16);
          packed[2] = o[4] | (o[5] << 16); packed[3] = o[6] | (o[7] << 16);
          const uint32_t off = col_ok ? (uint32_t)((row * g.ldo + ecol) * 2) : kOutOfRange;
          __builtin_amdgcn_raw_buffer_store_b128(packed, cur.ro, (int)off, 0, 0);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t off = ecol + e < cur.cols ? (uint32_t)((row * g.ldo + ecol + e) * 2) : kOutOfRange;
            __builtin_amdgcn_raw_buffer_store_b16((uint16_t)o[e], cur.ro, (int)off, 0, 0);
          }
        }
      }
      __builtin_amdgcn_wave_barrier();  // the next round rewrites E
    }
    cur = nxt;
    first = false;
  }
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
  // offsets need a 256-row panel (operands and output) to span less than
  // 2 GiB.
  return ((uintptr_t)g.a % 16 == 0) && ((uintptr_t)g.w % 16 == 0) && (g.lda % 16 == 0) && (g.ldw % 16 == 0) &&
         (g.K % 16 == 0) && (int64_t)BM * g.lda < (1ll << 31) && (int64_t)BN * g.ldw < (1ll << 31) &&
         (int64_t)BM * g.ldo * 2 < (1ll << 31) && ((uintptr_t)g.out % 2 == 0) && g.N < (1 << 29);
}

template <int FA, int FW>
hipError_t launch_mfma(const GemmArgs& g, bool fp8_accumulate, hipStream_t stream) {
  const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
  const int T = tiles_m * tiles_n;
  const unsigned grid = (unsigned)min(T, cu_count());
  const bool vec = (g.N % 8 == 0) && (g.ldo % 8 == 0) && ((uintptr_t)g.out % 16 == 0);
  if (fp8_accumulate) {
    if (vec)
      gemm_mfma_kernel<false, true, FA, FW><<<grid, kThreads, 0, stream>>>(g, tiles_m, tiles_n);
    else
      gemm_mfma_kernel<false, false, FA, FW><<<grid, kThreads, 0, stream>>>(g, tiles_m, tiles_n);
  } else {
    if (vec)
      gemm_mfma_kernel<true, true, FA, FW><<<grid, kThreads, 0, stream>>>(g, tiles_m, tiles_n);
    else
      gemm_mfma_kernel<true, false, FA, FW><<<grid, kThreads, 0, stream>>>(g, tiles_m, tiles_n);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_mfma(const GemmArgs& g, bool fp8_accumulate, hipStream_t stream) {
  if (g.fmt_a == kE5M2)
    return g.fmt_w == kE5M2 ? launch_mfma<kE5M2, kE5M2>(g, fp8_accumulate, stream)
                            : launch_mfma<kE5M2, kE4M3>(g, fp8_accumulate, stream);
  return g.fmt_w == kE5M2 ? launch_mfma<kE4M3, kE5M2>(g, fp8_accumulate, stream)
                          : launch_mfma<kE4M3, kE4M3>(g, fp8_accumulate, stream);
}

}  // namespace fp8w8a8
