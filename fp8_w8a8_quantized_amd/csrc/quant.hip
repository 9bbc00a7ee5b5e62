// Activation / weight quantization kernels (gfx950).
//
// Dynamic per-tensor quantization ("Prototype FP8Linear W8A8 runtime
// quantization", opening post: activations are quantized per call): the
// scale is amax/448, so amax needs the whole tensor before any code can be
// written.  Small tensors (decode activations) run in one workgroup that
// reads the tensor, reduces, and quantizes the now cache-resident tensor.
// Large tensors (prefill) run two launches on the same stream: per-block
// maxima into the workspace, then every block folds those maxima (a few KiB,
// from L2) into the scale and quantizes its share.  No atomics, so results
// and timing are deterministic, and the workspace needs no reset.
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

__device__ __forceinline__ uint32_t unit_absmax(const QuantArgs& a, uint32_t u) {
  const uint32_t r = fastdiv(u, a.div_units);
  const uint32_t c0 = (u - r * a.units_per_row) * 8;
  const uint16_t* row = a.x + (int64_t)r * a.ld_x;
  if (a.vec && c0 + 8 <= a.cols) {
    return absmax_bits8(*reinterpret_cast<const v4i*>(row + c0));
  }
  uint32_t m = 0;
  for (uint32_t c = c0; c < c0 + 8 && c < a.cols; ++c) m = max(m, (uint32_t)row[c] & 0x7fffu);
  return m;
}

__device__ __forceinline__ void unit_quant(const QuantArgs& a, uint32_t u, float s) {
  const uint32_t r = fastdiv(u, a.div_units);
  const uint32_t c0 = (u - r * a.units_per_row) * 8;
  const uint16_t* row = a.x + (int64_t)r * a.ld_x;
  uint8_t* qrow = a.q + (int64_t)r * a.ld_q;
  if (a.vec && c0 + 8 <= a.cols) {
    uint2 v = quant8(*reinterpret_cast<const v4i*>(row + c0), s);
    *reinterpret_cast<uint2*>(qrow + c0) = v;
    return;
  }
  for (uint32_t c = c0; c < c0 + 8 && c < a.cols; ++c)
    qrow[c] = (uint8_t)quant1(bf16_to_f32(row[c]), s);
}

// One workgroup: amax, scale, quantize.
__global__ __launch_bounds__(1024) void quant_dynamic_single_kernel(QuantArgs a, float* scale_out) {
  __shared__ uint32_t red[16];
  uint32_t m = 0;
  for (uint32_t u = threadIdx.x; u < a.total_units; u += blockDim.x) m = max(m, unit_absmax(a, u));
  m = block_max_u32(m, red);
  const float s = scale_from_amax(bf16_to_f32(m));
  if (threadIdx.x == 0) *scale_out = s;
  for (uint32_t u = threadIdx.x; u < a.total_units; u += blockDim.x) unit_quant(a, u, s);
}

// Launch 1 of 2: per-block maxima of |x| (as bf16 magnitude bits).
__global__ __launch_bounds__(256) void absmax_partial_kernel(QuantArgs a, uint32_t* partial) {
  __shared__ uint32_t red[16];
  uint32_t m = 0;
  for (uint32_t u = blockIdx.x * blockDim.x + threadIdx.x; u < a.total_units; u += gridDim.x * blockDim.x)
    m = max(m, unit_absmax(a, u));
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
  for (uint32_t u = blockIdx.x * blockDim.x + threadIdx.x; u < a.total_units; u += gridDim.x * blockDim.x)
    unit_quant(a, u, s);
}

__global__ __launch_bounds__(256) void quant_static_kernel(QuantArgs a, const float* scale) {
  const float s = *scale;
  for (uint32_t u = blockIdx.x * blockDim.x + threadIdx.x; u < a.total_units; u += gridDim.x * blockDim.x)
    unit_quant(a, u, s);
}

// One workgroup per row: the row's own amax and scale, then its codes.
__global__ __launch_bounds__(256) void quant_per_row_kernel(QuantArgs a, float* scales_out) {
  __shared__ uint32_t red[16];
  const uint32_t r = blockIdx.x;
  const uint32_t u0 = r * a.units_per_row, u1 = u0 + a.units_per_row;
  uint32_t m = 0;
  for (uint32_t u = u0 + threadIdx.x; u < u1; u += blockDim.x) m = max(m, unit_absmax(a, u));
  m = block_max_u32(m, red);
  const float s = scale_from_amax(bf16_to_f32(m));
  if (threadIdx.x == 0) scales_out[r] = s;
  for (uint32_t u = u0 + threadIdx.x; u < u1; u += blockDim.x) unit_quant(a, u, s);
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

constexpr uint32_t kPartialBlocks = 1024;       // max blocks of the two-launch path
constexpr uint32_t kSingleBlockUnits = 1u << 13;  // <= 64 Ki elements: one workgroup

uint32_t grid_for_units(uint32_t units, uint32_t cap) {
  uint32_t g = (units + 255) / 256;
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
  if (a.total_units <= kSingleBlockUnits) {
    quant_dynamic_single_kernel<<<1, 1024, 0, stream>>>(a, scale_out);
    return hipGetLastError();
  }
  uint32_t* partial = static_cast<uint32_t*>(workspace);
  const uint32_t grid = grid_for_units(a.total_units, kPartialBlocks);
  absmax_partial_kernel<<<grid, 256, 0, stream>>>(a, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const uint32_t grid2 = grid_for_units(a.total_units, 4096);
  quant_from_partial_kernel<<<grid2, 256, 0, stream>>>(a, partial, grid, scale_out);
  return hipGetLastError();
}

hipError_t launch_quant_static(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, const float* scale,
                               uint8_t* q, int64_t ld_q, hipStream_t stream) {
  if (rows == 0 || cols == 0) return hipSuccess;
  QuantArgs a = make_args(x, rows, cols, ld_x, q, ld_q);
  quant_static_kernel<<<grid_for_units(a.total_units, 4096), 256, 0, stream>>>(a, scale);
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
