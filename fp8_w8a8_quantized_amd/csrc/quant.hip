// Activation / weight quantization kernels (gfx950).
//
// Dynamic per-tensor quantization ("Prototype FP8Linear W8A8 runtime
// quantization", opening post: activations are quantized per call): the
// scale is amax/448, so amax needs the whole tensor before any code can be
// written.
//   * Small tensors (decode activations, up to 128 Ki elements): one launch
//     of up to 32 workgroups.  Every workgroup reduces the whole tensor
//     itself (at most 256 KiB, served by L2 after the first touch), so no
//     workgroup waits for another, and quantizes only its own share, which
//     it kept in registers from that pass.  (Past that size the redundant
//     reads cost more than a second launch: measured 11.5 us against 6.8 us
//     for 16 x 14336.)
//   * Large tensors (prefill): two launches on the same stream -- per-block
//     maxima into the workspace, then every block folds those maxima (a few
//     KiB, from L2) into the scale and quantizes its share.
// No atomics and no inter-workgroup waiting: results and timing are
// deterministic and the workspace needs no reset.  Each thread keeps
// several 16-byte loads in flight (kUnroll), which is what HBM needs.
//
// The same machinery quantizes values produced on the fly (value sources,
// below): the plain activations, a unit-weight RMS normalization of a
// residual stream (after an optional residual add), or a gate-first
// SiLU*mul.  Producer and quantization then share one pass over the input,
// so the produced bf16 tensor never round-trips through memory; an optional
// copy can still be written, by the pass that writes the codes.
//
// Rows are handled as units of 8 elements (16 bytes of bf16 in, 8 bytes of
// e4m3fn out).  The vector path needs 16-byte aligned input rows and 8-byte
// aligned output rows; a row's ragged end and unaligned layouts use
// element-wise loads and stores.

#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace fp8w8a8 {

namespace {

// The codes side of a quantization: where the e4m3 codes go and the unit
// geometry (a unit is 8 consecutive columns of one row).
struct QuantArgs {
  uint8_t* q;
  int64_t ld_q;
  uint32_t rows, cols, units_per_row, total_units;
  FastDivU32 div_units;
  bool vec_q;  // 8-byte aligned code rows
};

constexpr int kUnroll = 4;

__device__ __forceinline__ void unit_coords(const QuantArgs& a, uint32_t u, uint32_t& r, uint32_t& c0) {
  r = fastdiv(u, a.div_units);
  c0 = (u - r * a.units_per_row) * 8;
}

template <int F>
__device__ __forceinline__ void unit_store(const QuantArgs& a, uint32_t r, uint32_t c0, v4i x, float s) {
  uint8_t* qrow = a.q + (int64_t)r * a.ld_q;
  const uint2 v = quant8<F>(x, s);
  if (a.vec_q && c0 + 8 <= a.cols) {
    *reinterpret_cast<uint2*>(qrow + c0) = v;
    return;
  }
  for (uint32_t c = c0; c < c0 + 8 && c < a.cols; ++c) {
    const uint32_t w = (c - c0) < 4 ? v.x : v.y;
    qrow[c] = (uint8_t)(w >> (8 * ((c - c0) & 3)));
  }
}

// 8 bf16 of a row starting at column c0 (columns past `cols` read as +0).
__device__ __forceinline__ v4i load8_bf16(const uint16_t* row, uint32_t c0, uint32_t cols, bool vec) {
  if (vec && c0 + 8 <= cols) return *reinterpret_cast<const v4i*>(row + c0);
  uint32_t h[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (uint32_t c = c0; c < c0 + 8 && c < cols; ++c) h[c - c0] = row[c];
  v4i v;
  v[0] = (int)(h[0] | (h[1] << 16)); v[1] = (int)(h[2] | (h[3] << 16));
  v[2] = (int)(h[4] | (h[5] << 16)); v[3] = (int)(h[6] | (h[7] << 16));
  return v;
}

__device__ __forceinline__ void store8_bf16(uint16_t* row, uint32_t c0, uint32_t cols, bool vec, v4i v) {
  if (vec && c0 + 8 <= cols) {
    *reinterpret_cast<v4i*>(row + c0) = v;
    return;
  }
  for (uint32_t c = c0; c < c0 + 8 && c < cols; ++c) {
    const uint32_t w = (uint32_t)v[(c - c0) >> 1];
    row[c] = (uint16_t)(((c - c0) & 1) ? (w >> 16) : (w & 0xffffu));
  }
}

__device__ __forceinline__ float bf16_at(v4i v, int i) {
  const uint32_t w = (uint32_t)v[i >> 1];
  return bf16_to_f32((i & 1) ? (w >> 16) : (w & 0xffffu));
}

// float64 -> bf16 bits, one round-to-nearest-even (no double rounding through
// float32): the value is rounded to a multiple of its bf16 step 2^k,
// k = max(e-8, -133), where 2^(e-1) <= |x| < 2^e; the result is a bf16 value,
// exact in float32.  The scalings by 2^-k and 2^k are exact (x * 2^-k has at
// most 8 integer bits), so no division is needed.  NaN stays NaN.
__device__ __forceinline__ uint32_t f64_to_bf16_rne(double x) {
  if (x != x) return 0x7fc0u;
  int e;
  (void)frexp(x, &e);
  const int k = max(e - 8, -133);
  const double r = ldexp(rint(ldexp(x, -k)), k);
  return __float_as_uint((float)r) >> 16;
}

__device__ __forceinline__ v4i pack8_bf16_f64(const double f[8]) {
  v4i v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = (int)(f64_to_bf16_rne(f[2 * i]) | (f64_to_bf16_rne(f[2 * i + 1]) << 16));
  return v;
}

__device__ __forceinline__ v4i pack8_bf16(const float f[8]) {
  v4i v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = (int)pack_bf16x2_rne(f[2 * i], f[2 * i + 1]);
  return v;
}

// ---- value sources: the bf16 values a quantization encodes, per unit.
// load() gives the unit's 8 values (columns past `cols` as +0); emit() may
// write them out and is called once per unit, by the pass that writes the
// unit's codes.

// The activations themselves.
// kUnitsPerThread: the units a thread handles in the two-launch path (cheap
// sources take several to keep loads in flight; costly ones one, to spread
// the arithmetic over the whole chip).
struct PlainSrc {
  static constexpr uint32_t kUnitsPerThread = 4;
  const uint16_t* x;
  int64_t ld;
  bool vec;  // 16-byte aligned rows
  __device__ __forceinline__ v4i load(const QuantArgs& a, uint32_t r, uint32_t c0) const {
    return load8_bf16(x + (int64_t)r * ld, c0, a.cols, vec);
  }
  __device__ __forceinline__ void emit(const QuantArgs&, uint32_t, uint32_t, v4i) const {}
};

// Unit-weight RMS normalization: y = bf16(h * inv_rms[row]) in float64,
// inv_rms from norm_rows_kernel.
struct NormSrc {
  static constexpr uint32_t kUnitsPerThread = 1;
  const uint16_t* h;
  int64_t ld_h;
  const double* inv_rms;
  uint16_t* y;  // optional copy of the normalized values
  int64_t ld_y;
  bool vec_h, vec_y;
  __device__ __forceinline__ v4i load(const QuantArgs& a, uint32_t r, uint32_t c0) const {
    const v4i hv = load8_bf16(h + (int64_t)r * ld_h, c0, a.cols, vec_h);
    const double g = inv_rms[r];
    double f[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = (double)bf16_at(hv, i) * g;
    return pack8_bf16_f64(f);
  }
  __device__ __forceinline__ void emit(const QuantArgs& a, uint32_t r, uint32_t c0, v4i v) const {
    if (y != nullptr) store8_bf16(y + (int64_t)r * ld_y, c0, a.cols, vec_y, v);
  }
};

// bf16(g / (1 + exp(-g)) * u) as evaluated in float64 and rounded once,
// computed in float32 where that provably gives the same bf16.  The float32
// value (expf within 1 ulp, the add, v_rcp_f32 within 1 ulp, two multiplies:
// within 8 float32 ulps of the exact one for g > -80, where every
// intermediate is a normal number) rounds to the same bf16 as the exact
// value unless it lies within 8 ulps of a bf16 rounding midpoint, i.e.
// unless its low 16 bits are within 8 of 0x8000; there (with a margin of
// 32), for g <= -80 (expf nears overflow), and for results below 2^-100 the
// float64 expression decides.  That is about 0.1% of the values.
constexpr uint32_t kSiluMargin = 32;
__device__ __forceinline__ uint32_t silu_mul_bf16(float g, float u) {
  const float y = g * __builtin_amdgcn_rcpf(1.0f + expf(-g)) * u;
  const uint32_t low = __float_as_uint(y) & 0xffffu;
  const bool near_mid = low - (0x8000u - kSiluMargin) <= 2 * kSiluMargin;
  const bool tiny = fabsf(y) < 0x1p-100f && g != 0.0f && u != 0.0f;
  if (!(g > -80.0f) || near_mid || tiny) {
    const double gd = g;
    return f64_to_bf16_rne(gd / (1.0 + exp(-gd)) * (double)u);
  }
  return f32_to_bf16_rne(y);
}

// Gated activation, gate half first: y = bf16(silu(g) * u) with
// silu(g) = g / (1 + exp(-g)), the float64 value rounded once to bf16.
// FAST: through silu_mul_bf16 (same bits).  Measured at a prefill size
// (16384 x 14336) the quantization takes 627 us with it and 968 us without;
// at a decode size (16 x 14336), where the float64 branches of a few lanes
// hold up whole waves, 8.6 us with it and 7.8 us without.
template <bool FAST>
struct SiluMulSrc {
  static constexpr uint32_t kUnitsPerThread = 1;
  const uint16_t* gu;  // row r: gate columns [0, cols), up columns [cols, 2 cols)
  int64_t ld;
  uint16_t* y;  // optional copy of the activated values
  int64_t ld_y;
  bool vec, vec_y;
  __device__ __forceinline__ v4i load(const QuantArgs& a, uint32_t r, uint32_t c0) const {
    const uint16_t* row = gu + (int64_t)r * ld;
    const v4i gv = load8_bf16(row, c0, a.cols, vec);
    const v4i uv = load8_bf16(row + a.cols, c0, a.cols, vec);
    if constexpr (FAST) {
      uint32_t o[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = silu_mul_bf16(bf16_at(gv, i), bf16_at(uv, i));
      v4i v;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = (int)(o[2 * i] | (o[2 * i + 1] << 16));
      return v;
    } else {
      double f[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const double g = bf16_at(gv, i);
        f[i] = g / (1.0 + exp(-g)) * (double)bf16_at(uv, i);
      }
      return pack8_bf16_f64(f);
    }
  }
  __device__ __forceinline__ void emit(const QuantArgs& a, uint32_t r, uint32_t c0, v4i v) const {
    if (y != nullptr) store8_bf16(y + (int64_t)r * ld_y, c0, a.cols, vec_y, v);
  }
};

// max |x| bits over units u0, u0 + stride, ... < u1, UNROLL loads in flight
// N units u, u + stride, ... of a plain bf16 source with aligned rows and
// cols % 8 == 0: offsets first, then N unconditional buffer loads back to
// back (units at or past u1 get an out-of-range offset and read zeros).
template <int N>
__device__ __forceinline__ void load_units_buf(const QuantArgs& a, const PlainSrc& src, uint32_t u, uint32_t u1,
                                               uint32_t stride, v4i (&v)[N], uint32_t (&r)[N], uint32_t (&c0)[N]) {
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      (void*)src.x, (short)0, (int)(((int64_t)(a.rows - 1) * src.ld + a.cols) * 2), kRsrcWord3);
  uint32_t off[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const uint32_t uu = u + i * stride;
    unit_coords(a, uu, r[i], c0[i]);
    off[i] = uu < u1 ? (uint32_t)((r[i] * (uint32_t)src.ld + c0[i]) * 2) : kOutOfRange;
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < N; ++i)
    v[i] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rx, (int)off[i], 0, 0));
}

template <class Src, bool BUF = false, int UNROLL = kUnroll>
__device__ __forceinline__ uint32_t absmax_range(const QuantArgs& a, const Src& src, uint32_t u0, uint32_t u1,
                                                 uint32_t stride) {
  uint32_t m = 0;
  for (uint32_t u = u0; u < u1; u += stride * UNROLL) {
    v4i v[UNROLL];
    if constexpr (BUF) {
      uint32_t r[UNROLL], c0[UNROLL];
      load_units_buf<UNROLL>(a, src, u, u1, stride, v, r, c0);
    } else {
#pragma unroll
      for (int i = 0; i < UNROLL; ++i) {
        const uint32_t uu = u + i * stride;
        v[i] = v4i{0, 0, 0, 0};
        if (uu < u1) {
          uint32_t r, c0;
          unit_coords(a, uu, r, c0);
          v[i] = src.load(a, r, c0);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < UNROLL; ++i) m = max(m, absmax_bits8(v[i]));
  }
  return m;
}

template <int F, class Src, bool BUF = false>
__device__ __forceinline__ void quant_range(const QuantArgs& a, const Src& src, uint32_t u0, uint32_t u1,
                                            uint32_t stride, float s) {
  for (uint32_t u = u0; u < u1; u += stride * kUnroll) {
    v4i v[kUnroll];
    uint32_t r[kUnroll], c0[kUnroll];
    if constexpr (BUF) {
      load_units_buf<kUnroll>(a, src, u, u1, stride, v, r, c0);
    } else {
#pragma unroll
      for (int i = 0; i < kUnroll; ++i) {
        const uint32_t uu = u + i * stride;
        r[i] = 0; c0[i] = 0; v[i] = v4i{0, 0, 0, 0};
        if (uu < u1) {
          unit_coords(a, uu, r[i], c0[i]);
          v[i] = src.load(a, r[i], c0[i]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < kUnroll; ++i)
      if (u + i * stride < u1) {
        src.emit(a, r[i], c0[i], v[i]);
        unit_store<F>(a, r[i], c0[i], v[i], s);
      }
  }
}

// Small tensors, one launch: every workgroup reduces the whole tensor (512
// threads, 16 loads of 16 bytes in flight each), keeping in registers the
// slot it will quantize -- units blockIdx.x * 512 + threadIdx.x -- so the
// codes need no second read.  The grid has one workgroup per slot (at most
// 32); workgroup 0 writes the scale.  (Measured on the 16 x 4096 decode
// input: 4.3 us per launch with the buffer-load batches below, 5.1 us with
// a conditional load per unit, 5.4 us with 1024 threads x 8 loads.)
// Only for cheap sources: every workgroup evaluates the source over the
// whole tensor.
constexpr int kSmallThreads = 512;
constexpr int kSmallBatch = 16;
// BUF (plain bf16 source, 16-byte aligned rows, cols % 8 == 0, the tensor
// under 2 GiB): the batch's offsets are computed first and its 16 loads go
// out back to back as unconditional buffer loads (units past the end get an
// out-of-range offset and read zeros), one wait for all of them.  With a
// conditional load per unit the compiler waited for each in turn.
template <int F, class Src, bool BUF>
__global__ __launch_bounds__(kSmallThreads) void quant_dynamic_small_kernel(QuantArgs a, Src src, float* scale_out) {
  __shared__ uint32_t red[16];
  const uint32_t T = a.total_units;
  const uint32_t slots = gridDim.x;
  uint32_t m = 0;
  v4i keep = {0, 0, 0, 0};
  for (uint32_t j0 = 0; j0 < slots; j0 += kSmallBatch) {
    v4i v[kSmallBatch];
    if constexpr (BUF) {
      const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
          (void*)src.x, (short)0, (int)(((int64_t)(a.rows - 1) * src.ld + a.cols) * 2), kRsrcWord3);
      uint32_t off[kSmallBatch];
#pragma unroll
      for (int i = 0; i < kSmallBatch; ++i) {
        const uint32_t u = threadIdx.x + (j0 + i) * kSmallThreads;
        uint32_t r, c0;
        unit_coords(a, u, r, c0);
        off[i] = u < T ? (uint32_t)((r * (uint32_t)src.ld + c0) * 2) : kOutOfRange;
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < kSmallBatch; ++i)
        v[i] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rx, (int)off[i], 0, 0));
    } else {
#pragma unroll
      for (int i = 0; i < kSmallBatch; ++i) {
        const uint32_t u = threadIdx.x + (j0 + i) * kSmallThreads;
        v[i] = v4i{0, 0, 0, 0};
        if (u < T) {
          uint32_t r, c0;
          unit_coords(a, u, r, c0);
          v[i] = src.load(a, r, c0);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < kSmallBatch; ++i) {
      m = max(m, absmax_bits8(v[i]));
      if (j0 + i == blockIdx.x) keep = v[i];
    }
  }
  m = block_max_u32(m, red);
  const float s = scale_from_amax<F>(bf16_to_f32(m));
  if (blockIdx.x == 0 && threadIdx.x == 0) *scale_out = s;
  const uint32_t u = threadIdx.x + blockIdx.x * kSmallThreads;
  if (u < T) {
    uint32_t r, c0;
    unit_coords(a, u, r, c0);
    src.emit(a, r, c0, keep);
    unit_store<F>(a, r, c0, keep, s);
  }
}

// Launch 1 of 2: per-block maxima of |x| (as bf16 magnitude bits).
template <class Src, bool BUF = false>
__global__ __launch_bounds__(256) void absmax_partial_kernel(QuantArgs a, Src src, uint32_t* partial) {
  __shared__ uint32_t red[16];
  uint32_t m = absmax_range<Src, BUF>(a, src, blockIdx.x * blockDim.x + threadIdx.x, a.total_units,
                                      gridDim.x * blockDim.x);
  m = block_max_u32(m, red);
  if (threadIdx.x == 0) partial[blockIdx.x] = m;
}

// Launch 2 of 2: fold the maxima, derive the scale, quantize.
template <int F, class Src, bool BUF = false>
__global__ __launch_bounds__(256) void quant_from_partial_kernel(QuantArgs a, Src src, const uint32_t* partial,
                                                                  uint32_t nparts, float* scale_out) {
  __shared__ uint32_t red[16];
  uint32_t m = 0;
  for (uint32_t i = threadIdx.x; i < nparts; i += blockDim.x) m = max(m, partial[i]);
  m = block_max_u32(m, red);
  const float s = scale_from_amax<F>(bf16_to_f32(m));
  if (blockIdx.x == 0 && threadIdx.x == 0) *scale_out = s;
  quant_range<F, Src, BUF>(a, src, blockIdx.x * blockDim.x + threadIdx.x, a.total_units, gridDim.x * blockDim.x, s);
}

template <int F>
__global__ __launch_bounds__(256) void quant_static_kernel(QuantArgs a, PlainSrc src, const float* scale) {
  const float s = *scale;
  quant_range<F>(a, src, blockIdx.x * blockDim.x + threadIdx.x, a.total_units, gridDim.x * blockDim.x, s);
}

// One workgroup per row at a time (rows b, b + gridDim.x, ...): the row's
// own amax and scale, then its codes.
template <int F>
__global__ __launch_bounds__(256) void quant_per_row_kernel(QuantArgs a, PlainSrc src, float* scales_out) {
  __shared__ uint32_t red[16];
  for (uint32_t r = blockIdx.x; r < a.rows; r += gridDim.x) {
    const uint32_t u0 = r * a.units_per_row, u1 = u0 + a.units_per_row;
    uint32_t m = absmax_range(a, src, u0 + threadIdx.x, u1, blockDim.x);
    m = block_max_u32(m, red);
    const float s = scale_from_amax<F>(bf16_to_f32(m));
    if (threadIdx.x == 0) scales_out[r] = s;
    quant_range<F>(a, src, u0 + threadIdx.x, u1, blockDim.x, s);
  }
}

// Residual add, RMS statistics and the absmax of the normalized values, for
// rows b, b + gridDim.x, ... of workgroup b.  Per row: h' = bf16(h + d)
// (float32 add, one rounding; written to h_out when d is given), then
// inv_rms[row] = 1 / sqrt(sum(h'^2) / cols + eps) in float64 (the sum runs in
// a fixed order: per-thread units in order, then a fixed butterfly and wave
// order, so it is deterministic), then max |y| over y = bf16(h' * inv_rms).
// The float64 -> bf16 rounding is monotone and symmetric, so that maximum is
// the rounding of the row's largest |h'| times inv_rms: y is not evaluated
// here.  partial[b] = the workgroup's max, as bf16 magnitude bits: the
// quantization pass folds these maxima and evaluates every y once.
__global__ __launch_bounds__(256) void norm_rows_kernel(const uint16_t* h, int64_t ld_h, const uint16_t* d,
                                                        int64_t ld_d, uint16_t* h_out, int64_t ld_ho, uint32_t rows,
                                                        uint32_t cols, uint32_t units_per_row, double eps, bool vec,
                                                        double* inv_rms, uint32_t* partial) {
  __shared__ double wsum[4];
  __shared__ uint32_t wmax[4];
  __shared__ uint32_t red[16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t m = 0;
  for (uint32_t r = blockIdx.x; r < rows; r += gridDim.x) {
    const uint16_t* hrow = h + (int64_t)r * ld_h;
    const uint16_t* drow = d ? d + (int64_t)r * ld_d : nullptr;
    uint16_t* orow = d ? h_out + (int64_t)r * ld_ho : nullptr;
    double acc = 0.0;
    uint32_t hmax = 0;  // largest |h'| of the row, as bf16 magnitude bits
    for (uint32_t u = threadIdx.x; u < units_per_row; u += blockDim.x) {
      const uint32_t c0 = u * 8;
      v4i hv = load8_bf16(hrow, c0, cols, vec);
      if (drow != nullptr) {
        const v4i dv = load8_bf16(drow, c0, cols, vec);
        float f[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = bf16_at(hv, i) + bf16_at(dv, i);
        hv = pack8_bf16(f);
        store8_bf16(orow, c0, cols, vec, hv);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const double x = bf16_at(hv, i);
        acc = __builtin_fma(x, x, acc);
      }
      hmax = max(hmax, absmax_bits8(hv));
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    hmax = wave_max_u32(hmax);
    if (lane == 0) {
      wsum[wave] = acc;
      wmax[wave] = hmax;
    }
    __syncthreads();
    double t = 0.0;
    uint32_t hm = 0;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) {
      t += wsum[w];
      hm = max(hm, wmax[w]);
    }
    const double g = 1.0 / sqrt(t / (double)cols + eps);
    if (threadIdx.x == 0) inv_rms[r] = g;
    m = max(m, f64_to_bf16_rne((double)bf16_to_f32(hm) * g) & 0x7fffu);
    __syncthreads();  // wsum and wmax are rewritten for the next row
  }
  m = block_max_u32(m, red);
  if (threadIdx.x == 0) partial[blockIdx.x] = m;
}

__global__ void write_scale_kernel(float* scale_out, float v) { *scale_out = v; }

__global__ void fill_scales_kernel(float* scales, uint32_t n, float v) {
  uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) scales[i] = v;
}

QuantArgs make_args(int64_t rows, int64_t cols, uint8_t* q, int64_t ld_q) {
  QuantArgs a;
  a.q = q;
  a.ld_q = ld_q;
  a.rows = (uint32_t)rows;
  a.cols = (uint32_t)cols;
  a.units_per_row = (uint32_t)((cols + 7) / 8);
  a.total_units = a.rows * a.units_per_row;
  a.div_units = make_fastdiv(a.units_per_row);
  a.vec_q = ((uintptr_t)q % 8 == 0) && (ld_q % 8 == 0);
  return a;
}

bool rows16(const void* p, int64_t ld) { return ((uintptr_t)p % 16 == 0) && (ld % 8 == 0); }

PlainSrc plain_src(const uint16_t* x, int64_t ld_x) { return PlainSrc{x, ld_x, rows16(x, ld_x)}; }

constexpr uint32_t kPartialBlocks = 1024;         // max blocks of the two-launch path
constexpr uint32_t kSmallUnits = 1u << 14;        // <= 128 Ki elements (256 KiB): one launch
constexpr uint32_t kPerRowBlocks = 1u << 20;      // max blocks of the per-row quantization

uint32_t grid_for_units(uint32_t units, uint32_t per_block, uint32_t cap) {
  uint32_t g = (units + per_block - 1) / per_block;
  return g < 1 ? 1 : (g > cap ? cap : g);
}

// Dynamic per-tensor quantization of any source: one launch for small
// tensors of cheap sources, else two (per-block maxima in the workspace).
template <int F, class Src>
hipError_t launch_dynamic(const QuantArgs& a, const Src& src, bool small_ok, float* scale_out, void* workspace,
                          hipStream_t stream) {
  if (small_ok && a.total_units <= kSmallUnits) {
    // one workgroup per 512-unit slot: at most kSmallUnits / 512 = 32
    const uint32_t grid = (a.total_units + kSmallThreads - 1) / kSmallThreads;
    if constexpr (std::is_same<Src, PlainSrc>::value) {
      if (src.vec && a.cols % 8 == 0 && (int64_t)a.rows * src.ld * 2 < (int64_t(1) << 31)) {
        quant_dynamic_small_kernel<F, Src, true><<<grid, kSmallThreads, 0, stream>>>(a, src, scale_out);
        return hipGetLastError();
      }
    }
    quant_dynamic_small_kernel<F, Src, false><<<grid, kSmallThreads, 0, stream>>>(a, src, scale_out);
    return hipGetLastError();
  }
  uint32_t* partial = static_cast<uint32_t*>(workspace);
  const uint32_t grid = grid_for_units(a.total_units, 256 * Src::kUnitsPerThread, kPartialBlocks);
  const uint32_t grid2 = grid_for_units(a.total_units, 256 * Src::kUnitsPerThread, 8192);
  if constexpr (std::is_same<Src, PlainSrc>::value) {
    if (src.vec && a.cols % 8 == 0 && (int64_t)a.rows * src.ld * 2 < (int64_t(1) << 31)) {
      absmax_partial_kernel<Src, true><<<grid, 256, 0, stream>>>(a, src, partial);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      quant_from_partial_kernel<F, Src, true><<<grid2, 256, 0, stream>>>(a, src, partial, grid, scale_out);
      return hipGetLastError();
    }
  }
  absmax_partial_kernel<Src><<<grid, 256, 0, stream>>>(a, src, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  quant_from_partial_kernel<F, Src><<<grid2, 256, 0, stream>>>(a, src, partial, grid, scale_out);
  return hipGetLastError();
}

}  // namespace

size_t quant_workspace_bytes() { return kPartialBlocks * sizeof(uint32_t); }

// Shapes were validated by the caller: 0 <= rows, cols; rows*cols/8 < 2^31.
hipError_t launch_quant_dynamic(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, int fmt, uint8_t* q,
                                int64_t ld_q, float* scale_out, void* workspace, hipStream_t stream) {
  if (rows == 0 || cols == 0) {
    write_scale_kernel<<<1, 1, 0, stream>>>(scale_out, 1.0f);
    return hipGetLastError();
  }
  const QuantArgs a = make_args(rows, cols, q, ld_q);
  if (fmt == kE5M2) return launch_dynamic<kE5M2>(a, plain_src(x, ld_x), true, scale_out, workspace, stream);
  return launch_dynamic<kE4M3>(a, plain_src(x, ld_x), true, scale_out, workspace, stream);
}

size_t norm_quant_workspace_bytes(int64_t rows) {
  return quant_workspace_bytes() + (size_t)((rows * 8 + 255) / 256 * 256);
}

hipError_t launch_add_rmsnorm_quant(const uint16_t* h, int64_t ld_h, const uint16_t* delta, int64_t ld_delta,
                                    uint16_t* h_out, int64_t ld_h_out, int64_t rows, int64_t cols, float eps,
                                    uint16_t* y_out, int64_t ld_y, uint8_t* q, int64_t ld_q, float* scale_out,
                                    void* workspace, hipStream_t stream) {
  if (rows == 0 || cols == 0) {
    write_scale_kernel<<<1, 1, 0, stream>>>(scale_out, 1.0f);
    return hipGetLastError();
  }
  uint32_t* partial = static_cast<uint32_t*>(workspace);
  double* inv_rms = reinterpret_cast<double*>(static_cast<uint8_t*>(workspace) + quant_workspace_bytes());
  const bool vec = rows16(h, ld_h) && (delta == nullptr || (rows16(delta, ld_delta) && rows16(h_out, ld_h_out)));
  const QuantArgs a = make_args(rows, cols, q, ld_q);
  // launch 1: residual add, inv_rms and per-workgroup maxima of |y|
  const uint32_t groups = (uint32_t)min(rows, (int64_t)kPartialBlocks);
  norm_rows_kernel<<<groups, 256, 0, stream>>>(h, ld_h, delta, ld_delta, h_out, ld_h_out, (uint32_t)rows,
                                               (uint32_t)cols, a.units_per_row, (double)eps, vec, inv_rms, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // launch 2: fold the maxima into the scale, quantize (y evaluated again)
  const uint16_t* hs = delta ? h_out : h;
  const int64_t ld_hs = delta ? ld_h_out : ld_h;
  const NormSrc src{hs, ld_hs, inv_rms, y_out, ld_y, rows16(hs, ld_hs), y_out != nullptr && rows16(y_out, ld_y)};
  const uint32_t grid2 = grid_for_units(a.total_units, 256 * NormSrc::kUnitsPerThread, 8192);
  quant_from_partial_kernel<kE4M3, NormSrc><<<grid2, 256, 0, stream>>>(a, src, partial, groups, scale_out);
  return hipGetLastError();
}

hipError_t launch_silu_mul_quant(const uint16_t* gu, int64_t ld_gu, int64_t rows, int64_t cols, uint16_t* y_out,
                                 int64_t ld_y, uint8_t* q, int64_t ld_q, float* scale_out, void* workspace,
                                 hipStream_t stream) {
  if (rows == 0 || cols == 0) {
    write_scale_kernel<<<1, 1, 0, stream>>>(scale_out, 1.0f);
    return hipGetLastError();
  }
  // the up half starts at column cols: aligned only if cols % 8 == 0
  const bool vec = rows16(gu, ld_gu) && (cols % 8 == 0), vec_y = y_out != nullptr && rows16(y_out, ld_y);
  const QuantArgs a = make_args(rows, cols, q, ld_q);
  // the activation is costly to evaluate: never the redundant one-launch path
  if (rows * cols >= (int64_t(1) << 22))
    return launch_dynamic<kE4M3>(a, SiluMulSrc<true>{gu, ld_gu, y_out, ld_y, vec, vec_y}, false, scale_out,
                                 workspace, stream);
  return launch_dynamic<kE4M3>(a, SiluMulSrc<false>{gu, ld_gu, y_out, ld_y, vec, vec_y}, false, scale_out,
                               workspace, stream);
}

hipError_t launch_quant_static(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, int fmt,
                               const float* scale, uint8_t* q, int64_t ld_q, hipStream_t stream) {
  if (rows == 0 || cols == 0) return hipSuccess;
  QuantArgs a = make_args(rows, cols, q, ld_q);
  const uint32_t grid = grid_for_units(a.total_units, 256 * kUnroll, 8192);
  if (fmt == kE5M2)
    quant_static_kernel<kE5M2><<<grid, 256, 0, stream>>>(a, plain_src(x, ld_x), scale);
  else
    quant_static_kernel<kE4M3><<<grid, 256, 0, stream>>>(a, plain_src(x, ld_x), scale);
  return hipGetLastError();
}

hipError_t launch_quant_per_row(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, int fmt, uint8_t* q,
                                int64_t ld_q, float* scales_out, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  if (cols == 0) {
    fill_scales_kernel<<<(uint32_t)((rows + 255) / 256), 256, 0, stream>>>(scales_out, (uint32_t)rows, 1.0f);
    return hipGetLastError();
  }
  QuantArgs a = make_args(rows, cols, q, ld_q);
  // a launch's threads must stay below 2^32: past 2^20 rows the workgroups
  // take several rows each
  const uint32_t grid = (uint32_t)min(rows, (int64_t)kPerRowBlocks);
  if (fmt == kE5M2)
    quant_per_row_kernel<kE5M2><<<grid, 256, 0, stream>>>(a, plain_src(x, ld_x), scales_out);
  else
    quant_per_row_kernel<kE4M3><<<grid, 256, 0, stream>>>(a, plain_src(x, ld_x), scales_out);
  return hipGetLastError();
}

}  // namespace fp8w8a8
