// Activation / weight quantization kernels (gfx950).
//
// Dynamic per-tensor quantization ("Prototype FP8Linear W8A8 runtime
// quantization", opening post: activations are quantized per call): the
// scale is amax/448, so amax needs the whole tensor before any code can be
// written.
//   * Small tensors (decode activations, up to 256 Ki elements): one launch
//     of up to 32 workgroups.  Every workgroup reduces the whole tensor
//     itself (at most 512 KiB, served by L2 after the first touch), so no
//     workgroup waits for another, and quantizes only its own share, which
//     it kept in registers from that pass.
//   * Large tensors (prefill): two launches on the same stream -- per-block
//     maxima into the workspace, then every block folds those maxima (a few
//     KiB, from L2) into the scale and quantizes its share.
// No atomics and no inter-workgroup waiting: results and timing are
// deterministic and the workspace needs no reset.  Each thread keeps
// several 16-byte loads in flight (kUnroll), which is what HBM needs.
//
// Rows are handled as units of 8 elements (16 bytes of bf16 in, 8 bytes of
// e4m3fn out).  The vector path needs 16-byte aligned input rows and 8-byte
// aligned output rows; a row's ragged end and unaligned layouts use
// element-wise loads and stores.

#include "device_common.h"
#include "internal.h"

namespace fp8w8a8 {

namespace {

struct QuantArgs {
  const uint16_t* x;
  uint8_t* q;
  int64_t ld_x, ld_q;
  uint32_t rows, cols, units_per_row, total_units;
  FastDivU32 div_units;
  bool vec;  // aligned layout: 16-byte input rows, 8-byte output rows
};

constexpr int kUnroll = 4;

__device__ __forceinline__ bool unit_is_vector(const QuantArgs& a, uint32_t c0) {
  return a.vec && c0 + 8 <= a.cols;
}

__device__ __forceinline__ void unit_coords(const QuantArgs& a, uint32_t u, uint32_t& r, uint32_t& c0) {
  r = fastdiv(u, a.div_units);
  c0 = (u - r * a.units_per_row) * 8;
}

__device__ __forceinline__ v4i unit_load(const QuantArgs& a, uint32_t r, uint32_t c0) {
  const uint16_t* row = a.x + (int64_t)r * a.ld_x;
  if (unit_is_vector(a, c0)) return *reinterpret_cast<const v4i*>(row + c0);
  uint32_t h[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (uint32_t c = c0; c < c0 + 8 && c < a.cols; ++c) h[c - c0] = row[c];
  v4i v;
  v[0] = (int)(h[0] | (h[1] << 16)); v[1] = (int)(h[2] | (h[3] << 16));
  v[2] = (int)(h[4] | (h[5] << 16)); v[3] = (int)(h[6] | (h[7] << 16));
  return v;  // missing elements are +0 and do not change the max
}

__device__ __forceinline__ void unit_store(const QuantArgs& a, uint32_t r, uint32_t c0, v4i x, float s) {
  uint8_t* qrow = a.q + (int64_t)r * a.ld_q;
  const uint2 v = quant8(x, s);
  if (unit_is_vector(a, c0)) {
    *reinterpret_cast<uint2*>(qrow + c0) = v;
    return;
  }
  for (uint32_t c = c0; c < c0 + 8 && c < a.cols; ++c) {
    const uint32_t w = (c - c0) < 4 ? v.x : v.y;
    qrow[c] = (uint8_t)(w >> (8 * ((c - c0) & 3)));
  }
}

// max |x| bits over units u0, u0 + stride, ... < u1, UNROLL loads in flight
template <int UNROLL = kUnroll>
__device__ __forceinline__ uint32_t absmax_range(const QuantArgs& a, uint32_t u0, uint32_t u1, uint32_t stride) {
  uint32_t m = 0;
  for (uint32_t u = u0; u < u1; u += stride * UNROLL) {
    v4i v[UNROLL];
#pragma unroll
    for (int i = 0; i < UNROLL; ++i) {
      const uint32_t uu = u + i * stride;
      v[i] = v4i{0, 0, 0, 0};
      if (uu < u1) {
        uint32_t r, c0;
        unit_coords(a, uu, r, c0);
        v[i] = unit_load(a, r, c0);
      }
    }
#pragma unroll
    for (int i = 0; i < UNROLL; ++i) m = max(m, absmax_bits8(v[i]));
  }
  return m;
}

__device__ __forceinline__ void quant_range(const QuantArgs& a, uint32_t u0, uint32_t u1, uint32_t stride, float s) {
  for (uint32_t u = u0; u < u1; u += stride * kUnroll) {
    v4i v[kUnroll];
    uint32_t r[kUnroll], c0[kUnroll];
#pragma unroll
    for (int i = 0; i < kUnroll; ++i) {
      const uint32_t uu = u + i * stride;
      r[i] = 0; c0[i] = 0; v[i] = v4i{0, 0, 0, 0};
      if (uu < u1) {
        unit_coords(a, uu, r[i], c0[i]);
        v[i] = unit_load(a, r[i], c0[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < kUnroll; ++i)
      if (u + i * stride < u1) unit_store(a, r[i], c0[i], v[i], s);
  }
}

// Small tensors, one launch: every workgroup reduces the whole tensor (1024
// threads, 8 loads of 16 bytes in flight each), keeping in registers the
// slot it will quantize -- units blockIdx.x * 1024 + threadIdx.x -- so the
// codes need no second read.  The grid has one workgroup per slot (at most
// 32); workgroup 0 writes the scale.
constexpr int kSmallThreads = 1024;
constexpr int kSmallBatch = 8;
__global__ __launch_bounds__(kSmallThreads) void quant_dynamic_small_kernel(QuantArgs a, float* scale_out) {
  __shared__ uint32_t red[16];
  const uint32_t T = a.total_units;
  const uint32_t slots = gridDim.x;
  uint32_t m = 0;
  v4i keep = {0, 0, 0, 0};
  for (uint32_t j0 = 0; j0 < slots; j0 += kSmallBatch) {
    v4i v[kSmallBatch];
#pragma unroll
    for (int i = 0; i < kSmallBatch; ++i) {
      const uint32_t u = threadIdx.x + (j0 + i) * kSmallThreads;
      v[i] = v4i{0, 0, 0, 0};
      if (u < T) {
        uint32_t r, c0;
        unit_coords(a, u, r, c0);
        v[i] = unit_load(a, r, c0);
      }
    }
#pragma unroll
    for (int i = 0; i < kSmallBatch; ++i) {
      m = max(m, absmax_bits8(v[i]));
      if (j0 + i == blockIdx.x) keep = v[i];
    }
  }
  m = block_max_u32(m, red);
  const float s = scale_from_amax(bf16_to_f32(m));
  if (blockIdx.x == 0 && threadIdx.x == 0) *scale_out = s;
  const uint32_t u = threadIdx.x + blockIdx.x * kSmallThreads;
  if (u < T) {
    uint32_t r, c0;
    unit_coords(a, u, r, c0);
    unit_store(a, r, c0, keep, s);
  }
}

// Launch 1 of 2: per-block maxima of |x| (as bf16 magnitude bits).
__global__ __launch_bounds__(256) void absmax_partial_kernel(QuantArgs a, uint32_t* partial) {
  __shared__ uint32_t red[16];
  uint32_t m = absmax_range(a, blockIdx.x * blockDim.x + threadIdx.x, a.total_units, gridDim.x * blockDim.x);
  m = block_max_u32(m, red);
  if (threadIdx.x == 0) partial[blockIdx.x] = m;
}

// Launch 2 of 2: fold the maxima, derive the scale, quantize.
__global__ __launch_bounds__(256) void quant_from_partial_kernel(QuantArgs a, const uint32_t* partial,
                                                                  uint32_t nparts, float* scale_out) {
  __shared__ uint32_t red[16];
  uint32_t m = 0;
  for (uint32_t i = threadIdx.x; i < nparts; i += blockDim.x) m = max(m, partial[i]);
  m = block_max_u32(m, red);
  const float s = scale_from_amax(bf16_to_f32(m));
  if (blockIdx.x == 0 && threadIdx.x == 0) *scale_out = s;
  quant_range(a, blockIdx.x * blockDim.x + threadIdx.x, a.total_units, gridDim.x * blockDim.x, s);
}

__global__ __launch_bounds__(256) void quant_static_kernel(QuantArgs a, const float* scale) {
  const float s = *scale;
  quant_range(a, blockIdx.x * blockDim.x + threadIdx.x, a.total_units, gridDim.x * blockDim.x, s);
}

// One workgroup per row: the row's own amax and scale, then its codes.
__global__ __launch_bounds__(256) void quant_per_row_kernel(QuantArgs a, float* scales_out) {
  __shared__ uint32_t red[16];
  const uint32_t r = blockIdx.x;
  const uint32_t u0 = r * a.units_per_row, u1 = u0 + a.units_per_row;
  uint32_t m = absmax_range(a, u0 + threadIdx.x, u1, blockDim.x);
  m = block_max_u32(m, red);
  const float s = scale_from_amax(bf16_to_f32(m));
  if (threadIdx.x == 0) scales_out[r] = s;
  quant_range(a, u0 + threadIdx.x, u1, blockDim.x, s);
}

__global__ void write_scale_kernel(float* scale_out, float v) { *scale_out = v; }

__global__ void fill_scales_kernel(float* scales, uint32_t n, float v) {
  uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) scales[i] = v;
}

QuantArgs make_args(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* q, int64_t ld_q) {
  QuantArgs a;
  a.x = x;
  a.q = q;
  a.ld_x = ld_x;
  a.ld_q = ld_q;
  a.rows = (uint32_t)rows;
  a.cols = (uint32_t)cols;
  a.units_per_row = (uint32_t)((cols + 7) / 8);
  a.total_units = a.rows * a.units_per_row;
  a.div_units = make_fastdiv(a.units_per_row);
  a.vec = ((uintptr_t)x % 16 == 0) && (ld_x % 8 == 0) && ((uintptr_t)q % 8 == 0) && (ld_q % 8 == 0);
  return a;
}

constexpr uint32_t kPartialBlocks = 1024;         // max blocks of the two-launch path
constexpr uint32_t kSmallUnits = 1u << 15;        // <= 256 Ki elements (512 KiB): one launch

uint32_t grid_for_units(uint32_t units, uint32_t per_block, uint32_t cap) {
  uint32_t g = (units + per_block - 1) / per_block;
  return g < 1 ? 1 : (g > cap ? cap : g);
}

}  // namespace

size_t quant_workspace_bytes() { return kPartialBlocks * sizeof(uint32_t); }

// Shapes were validated by the caller: 0 <= rows, cols; rows*cols/8 < 2^32.
hipError_t launch_quant_dynamic(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* q,
                                int64_t ld_q, float* scale_out, void* workspace, hipStream_t stream) {
  if (rows == 0 || cols == 0) {
    write_scale_kernel<<<1, 1, 0, stream>>>(scale_out, 1.0f);
    return hipGetLastError();
  }
  QuantArgs a = make_args(x, rows, cols, ld_x, q, ld_q);
  if (a.total_units <= kSmallUnits) {
    // one workgroup per 1024-unit slot: at most kSmallUnits / 1024 = 32
    const uint32_t grid = (a.total_units + kSmallThreads - 1) / kSmallThreads;
    quant_dynamic_small_kernel<<<grid, kSmallThreads, 0, stream>>>(a, scale_out);
    return hipGetLastError();
  }
  uint32_t* partial = static_cast<uint32_t*>(workspace);
  const uint32_t grid = grid_for_units(a.total_units, 256 * kUnroll, kPartialBlocks);
  absmax_partial_kernel<<<grid, 256, 0, stream>>>(a, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const uint32_t grid2 = grid_for_units(a.total_units, 256 * kUnroll, 8192);
  quant_from_partial_kernel<<<grid2, 256, 0, stream>>>(a, partial, grid, scale_out);
  return hipGetLastError();
}

hipError_t launch_quant_static(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, const float* scale,
                               uint8_t* q, int64_t ld_q, hipStream_t stream) {
  if (rows == 0 || cols == 0) return hipSuccess;
  QuantArgs a = make_args(x, rows, cols, ld_x, q, ld_q);
  quant_static_kernel<<<grid_for_units(a.total_units, 256 * kUnroll, 8192), 256, 0, stream>>>(a, scale);
  return hipGetLastError();
}

hipError_t launch_quant_per_row(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* q,
                                int64_t ld_q, float* scales_out, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  if (cols == 0) {
    fill_scales_kernel<<<(uint32_t)((rows + 255) / 256), 256, 0, stream>>>(scales_out, (uint32_t)rows, 1.0f);
    return hipGetLastError();
  }
  QuantArgs a = make_args(x, rows, cols, ld_x, q, ld_q);
  quant_per_row_kernel<<<(uint32_t)rows, 256, 0, stream>>>(a, scales_out);
  return hipGetLastError();
}

}  // namespace fp8w8a8
