// Skinny-M scaled FP8 GEMM for decode (M <= 16), gfx950.
//
// "[WIP] FP8 support" (text-generation-inference PR 1484), review discussion:
// decode runs at fewer than 16 rows, wants a dedicated GEMV-like kernel, and
// must not pay for per-call packing or 16-padding.  Here the weight streams
// from HBM straight into the matrix cores' A operand, one 16-row slice of W
// per workgroup, each byte read once; the activation rows (at most 16) are
// the B operand, and rows >= M are zeros in registers, never in memory.
//
// Accumulation: the fp8 matrix-core instruction sums each group of 8
// products with only 13 bits below the group's largest product (measured on
// gfx950), which loses small products next to large ones.  This path is
// bound by HBM, not by the matrix cores, so it converts the e4m3 codes to
// bf16 in registers (exact: every e4m3 value is a bf16 value) and uses the
// bf16 instruction v_mfma_f32_16x16x32_bf16, whose sums keep fp32-class
// precision.  HBM traffic is unchanged: one byte per weight.
//
// Lane l holds row (l % 16) of each operand and 32 k-values of it per
// 128-wide k step, and both operands use the same lane/element -> k
// assignment, so products pair matching k whatever order the hardware sums
// in.  Lane group g = l / 16 takes bytes [16g, 16g+16) and
// [64+16g, 64+16g+16) of each 128-byte k step: every 16-byte load
// instruction then reads 64 contiguous bytes of each of 16 rows.
//
// The waves of a workgroup split the k steps (interleaved, so the group
// reads adjacent 128-byte blocks of a row together) and are summed through
// LDS in a fixed order, so results do not depend on timing.  The rescale
// epilogue out = acc * (s_a * s_w[n]) + bias[n] -> bf16 is applied in the
// store ("[Kernel] Implement fallback for FP8 channelwise using
// torch._scaled_mm", description: the channelwise rescale follows the
// per-tensor GEMM; fused here instead of a separate pass).
//
// Larger M runs the same kernel over a grid of 16-row blocks of M; that is
// the fallback for layouts the matrix-core GEMM does not take.

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

// 4 e4m3 codes (one 32-bit word) -> 4 bf16 values, exactly (scale 1).
__device__ __forceinline__ void e4m3x4_to_bf16(int w, bf16x8& dst, int at) {
  bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  dst[at] = lo[0]; dst[at + 1] = lo[1]; dst[at + 2] = hi[0]; dst[at + 3] = hi[1];
}

// acc += W_frag . A_frag over 32 e4m3 k-values per lane, as four bf16
// 16x16x32 products (k-values 8t..8t+7 of the lane feed instruction t).
__device__ __forceinline__ v4f mfma_e4m3_as_bf16(v8i wf, v8i af, v4f acc) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    bf16x8 wb, ab;
    e4m3x4_to_bf16(wf[2 * t], wb, 0);
    e4m3x4_to_bf16(wf[2 * t + 1], wb, 4);
    e4m3x4_to_bf16(af[2 * t], ab, 0);
    e4m3x4_to_bf16(af[2 * t + 1], ab, 4);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wb, ab, acc, 0, 0, 0);
  }
  return acc;
}

template <int NW, int U, bool VEC>
__global__ __launch_bounds__(NW * 64) void gemm_skinny_kernel(GemmArgs g) {
  __shared__ float red[NW][4][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 15, grp = lane >> 4;
  const int n0 = blockIdx.x * 16, m0 = blockIdx.y * 16;
  const bool n_ok = n0 + r < g.N, m_ok = m0 + r < g.M;
  const uint8_t* wrow = g.w + (int64_t)(n_ok ? n0 + r : 0) * g.ldw;
  const uint8_t* arow = g.a + (int64_t)(m_ok ? m0 + r : 0) * g.lda;
  const int ks = (g.K + 127) >> 7;

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
    for (int u = 0; u < U; ++u) acc = mfma_e4m3_as_bf16(wf[u], af[u], acc);
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) red[wave][i][lane] = acc[i];
  __syncthreads();
  if (wave != 0) return;
  float sum[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float t = red[0][i][lane];
#pragma unroll
    for (int w = 1; w < NW; ++w) t += red[w][i][lane];
    sum[i] = t;
  }

  // Result layout: lane holds output row m = m0 + (lane % 16) and the four
  // consecutive columns n = n0 + 4 * (lane / 16) + i.
  const int m = m0 + r;
  if (m >= g.M) return;
  const int nb = n0 + 4 * grp;
  const float sa = *g.s_a;
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int n = nb + i;
    if (n < g.N) {
      const float sc = sa * (g.per_channel ? g.s_w[n] : g.s_w[0]);
      const float b = g.bias ? bf16_to_f32(g.bias[n]) : 0.0f;
      o[i] = f32_to_bf16_rne(__builtin_fmaf(sum[i], sc, b));
    }
  }
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

template <int NW, bool VEC>
hipError_t launch_nw(const GemmArgs& g, dim3 grid, hipStream_t stream) {
  constexpr int U = NW >= 16 ? 4 : 8;  // 16 waves leave 128 VGPRs per lane
  gemm_skinny_kernel<NW, U, VEC><<<grid, NW * 64, 0, stream>>>(g);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_skinny(const GemmArgs& g, hipStream_t stream) {
  const bool vec = ((uintptr_t)g.a % 16 == 0) && ((uintptr_t)g.w % 16 == 0) && (g.lda % 16 == 0) &&
                   (g.ldw % 16 == 0) && (g.K % 16 == 0);
  const int64_t tiles_n = (g.N + 15) / 16, tiles_m = (g.M + 15) / 16;
  dim3 grid((unsigned)tiles_n, (unsigned)tiles_m);
  const int64_t tiles = tiles_n * tiles_m;
  const int ks = (g.K + 127) / 128;
  // More waves per workgroup when there are few workgroups, so that enough
  // weight bytes are in flight to cover HBM latency; never more waves than
  // k steps.
  int nw = tiles >= 256 ? 4 : (tiles >= 128 ? 8 : 16);
  while (nw > 1 && nw > ks) nw >>= 1;
  switch (nw) {
    case 16: return vec ? launch_nw<16, true>(g, grid, stream) : launch_nw<16, false>(g, grid, stream);
    case 8: return vec ? launch_nw<8, true>(g, grid, stream) : launch_nw<8, false>(g, grid, stream);
    case 4: return vec ? launch_nw<4, true>(g, grid, stream) : launch_nw<4, false>(g, grid, stream);
    case 2: return vec ? launch_nw<2, true>(g, grid, stream) : launch_nw<2, false>(g, grid, stream);
    default: return vec ? launch_nw<1, true>(g, grid, stream) : launch_nw<1, false>(g, grid, stream);
  }
}

}  // namespace fp8w8a8
