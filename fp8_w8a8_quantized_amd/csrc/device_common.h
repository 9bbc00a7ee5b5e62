// Device helpers shared by the gfx950 kernels of the FP8 W8A8 linear layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8w8a8 {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr float kE4M3Max = 448.0f;
constexpr float kE5M2Max = 57344.0f;

// fp8 formats: e4m3 (OCP E4M3, finite-only variant, the pages' format) and
// e5m2 (OCP E5M2, the extension named on the compressed-tensors fp8 page).
enum Fmt : int { kE4M3 = 0, kE5M2 = 1 };

template <int F>
__device__ __forceinline__ constexpr float fmt_max() {
  return F == kE5M2 ? kE5M2Max : kE4M3Max;
}

// s_waitcnt immediate for gfx9: lgkmcnt(0), vmcnt and expcnt left at max.
constexpr int kWaitLgkm0 = 0xC07F;
// s_waitcnt immediate for gfx9: vmcnt(0), expcnt and lgkmcnt left at max.
constexpr int kWaitVm0 = 0x0F70;
// s_waitcnt immediate for gfx9: vmcnt(n), 0 <= n < 64 (vmcnt bits 3:0 and
// 15:14), expcnt and lgkmcnt left at max.
constexpr int wait_vmcnt(int n) { return ((n >> 4) << 14) | 0x0F70 | (n & 15); }
static_assert(wait_vmcnt(0) == kWaitVm0 && wait_vmcnt(32) == 0x8F70, "s_waitcnt vmcnt encoding");

// Raw buffer resources (gfx9): word 3 selects the 32-bit data format.  A
// load whose byte offset reaches num_records returns zeros without touching
// memory; offsets at or above kOutOfRange are out of range for every
// resource these kernels build (num_records stays below 2^31).
constexpr int kRsrcWord3 = 0x00020000;
constexpr uint32_t kOutOfRange = 0x80000000u;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// float32 -> bf16 bits, round to nearest even: the language's conversion,
// which gfx950 performs with v_cvt_pk_bf16_f32 (two values per instruction).
// Measured on MI355X over all 2^32 float32 patterns: bit-identical to the
// integer rounding (u + 0x7fff + ((u >> 16) & 1)) >> 16 on every non-NaN
// input (denormals and infinities included); a NaN gives a NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Two float32 -> a packed bf16 pair (a in the low half), rounded as above.
__device__ __forceinline__ uint32_t pack_bf16x2_rne(float a, float b) {
  bf16x2 v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// Per-tensor scale from amax: amax / max(format) correctly rounded in
// float32; an all-zero tensor has no range to map and takes scale 1.
template <int F = kE4M3>
__device__ __forceinline__ float scale_from_amax(float amax) {
  return amax == 0.0f ? 1.0f : amax / fmt_max<F>();
}

// Two fp8 codes packed into byte pair `hi` of `old`: the hardware's fp8
// (e4m3) or bf8 (e5m2) conversion, both round to nearest even on gfx950.
template <int F, bool HI>
__device__ __forceinline__ uint32_t cvt_pk(float a, float b, uint32_t old) {
  if constexpr (F == kE5M2)
    return __builtin_amdgcn_cvt_pk_bf8_f32(a, b, old, HI);
  else
    return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, HI);
}

// Saturating round-to-nearest-even codes for four values divided by s.  The
// division is the correctly rounded float32 one (the compiler's default for
// '/'), then the quotient is clamped to +-max and converted by the hardware,
// which rounds to nearest even (OCP codes on gfx950) but does not saturate
// (e4m3: past 464 gives NaN; e5m2: past 61440 gives infinity) -- hence the
// clamp.
template <int F = kE4M3>
__device__ __forceinline__ uint32_t quant4(float a, float b, float c, float d, float s) {
  constexpr float M = fmt_max<F>();
  float qa = __builtin_amdgcn_fmed3f(a / s, -M, M);
  float qb = __builtin_amdgcn_fmed3f(b / s, -M, M);
  float qc = __builtin_amdgcn_fmed3f(c / s, -M, M);
  float qd = __builtin_amdgcn_fmed3f(d / s, -M, M);
  uint32_t w = cvt_pk<F, false>(qa, qb, 0);
  return cvt_pk<F, true>(qc, qd, w);
}

// Quantize 8 bf16 values packed in a 16-byte word into 8 fp8 bytes.
template <int F = kE4M3>
__device__ __forceinline__ uint2 quant8(v4i x, float s) {
  uint2 r;
  r.x = quant4<F>(bf16_to_f32(x[0] & 0xffff), bf16_to_f32((uint32_t)x[0] >> 16),
                  bf16_to_f32(x[1] & 0xffff), bf16_to_f32((uint32_t)x[1] >> 16), s);
  r.y = quant4<F>(bf16_to_f32(x[2] & 0xffff), bf16_to_f32((uint32_t)x[2] >> 16),
                  bf16_to_f32(x[3] & 0xffff), bf16_to_f32((uint32_t)x[3] >> 16), s);
  return r;
}

// 4 fp8 codes (one 32-bit word) -> 2 x 2 bf16 values, exactly (every e4m3
// and every finite e5m2 value is a bf16 value; the scale is 1).
template <int F, bool HI>
__device__ __forceinline__ bf16x2 fp8x2_to_bf16(int w) {
  if constexpr (F == kE5M2)
    return __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.0f, HI);
  else
    return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI);
}

// Largest |bf16| among 8 packed values, as the 15-bit magnitude pattern.
// For finite bf16 the magnitude bits order like the magnitudes themselves.
__device__ __forceinline__ uint32_t absmax_bits8(v4i x) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t w = (uint32_t)x[i];
    m = max(m, w & 0x7fffu);
    m = max(m, (w >> 16) & 0x7fffu);
  }
  return m;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
  return v;
}

// Block-wide max; every thread gets the result.  `red` holds >= 16 words.
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t* red) {
  v = wave_max_u32(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nwaves = (blockDim.x + 63) >> 6;
  __syncthreads();  // red may be in use by a previous call
  if (lane == 0) red[wave] = v;
  __syncthreads();
  uint32_t r = 0;
  for (int w = 0; w < nwaves; ++w) r = max(r, red[w]);
  return r;
}

// Exact unsigned 32-bit division by a run-time invariant divisor with one
// multiply-high, after Granlund and Montgomery, "Division by invariant
// integers using multiplication" (PLDI 1994), figure 4.1.
struct FastDivU32 {
  uint32_t d, m, s1, s2;
};

__host__ __device__ inline FastDivU32 make_fastdiv(uint32_t d) {
  FastDivU32 f;
  f.d = d;
  uint32_t l = 0;
  while (l < 32 && (1ull << l) < d) ++l;
  f.m = (uint32_t)((((1ull << l) - d) << 32) / d + 1);
  f.s1 = l < 1 ? l : 1;
  f.s2 = l > 0 ? l - 1 : 0;
  return f;
}

__device__ __forceinline__ uint32_t fastdiv(uint32_t n, const FastDivU32& f) {
  uint32_t t = __umulhi(f.m, n);
  return (t + ((n - t) >> f.s1)) >> f.s2;
}

}  // namespace fp8w8a8
