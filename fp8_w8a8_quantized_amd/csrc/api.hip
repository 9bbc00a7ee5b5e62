// C ABI of the FP8 W8A8 linear layer: host-side validation and dispatch.
// Every argument check runs before any HIP call, so invalid calls fail
// without touching the device (and work on machines without a GPU).

#include <stdio.h>
#include <stdarg.h>

#include <mutex>

#include "../../include/fp8w8a8.h"
#include "internal.h"

namespace {

thread_local char g_err[512] = "";

fp8_status fail(fp8_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

fp8_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return FP8_OK;
  return fail(FP8_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
}

// Shared checks of the quantization calls.  Element counts are capped so
// that units of 8 elements index in 32 bits.
fp8_status check_quant(const char* fn, const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                       const uint8_t* q, int64_t ld_q) {
  if (rows < 0 || cols < 0) return fail(FP8_ERR_INVALID_ARG, "%s: negative size (rows=%lld, cols=%lld)", fn,
                                        (long long)rows, (long long)cols);
  if (ld_x < cols || ld_q < cols)
    return fail(FP8_ERR_INVALID_ARG, "%s: leading dimension smaller than cols (ld_x=%lld, ld_q=%lld, cols=%lld)",
                fn, (long long)ld_x, (long long)ld_q, (long long)cols);
  if (rows > 0 && cols > 0 && (x == nullptr || q == nullptr))
    return fail(FP8_ERR_INVALID_ARG, "%s: null input or output pointer", fn);
  if (rows > 0 && cols > 0 && rows * ((cols + 7) / 8) >= (1ll << 31))
    return fail(FP8_ERR_UNSUPPORTED, "%s: tensor too large (rows=%lld, cols=%lld)", fn, (long long)rows,
                (long long)cols);
  return FP8_OK;
}

fp8_status check_fmt(const char* fn, fp8_format f) {
  if (f != FP8_FORMAT_E4M3 && f != FP8_FORMAT_E5M2) return fail(FP8_ERR_INVALID_ARG, "%s: unknown format %d", fn, (int)f);
  return FP8_OK;
}

// Up to 256 rows the matrix-core GEMM has at most 2 ceil(N / 128) tiles of
// 128 x 128 (one per CU at a time), so for N up to some 16k it runs a single
// round of tiles whose time is proportional to K whatever M and N: about 36
// us at K = 4096 with fp32-class sums, 29-33 us with fp8 sums.  The skinny
// kernel reads the weight once per grid row of up to 64 rows of M, in time
// about proportional to N and to the 16-row blocks each grid row carries
// (the blocks of M are spread evenly over the ceil(M / 64) grid rows: 65 to
// 96 rows run two rows of 3 blocks).  So the skinny kernel runs while
// N x (grid rows x blocks per row) < 81920, in both modes (it always sums
// with fp32-class precision).  Measured at K = 4096 and 14336 for N from
// 4096 to 14336 and M from 65 to 256, with weights from HBM: every choice
// within 2.1% of the faster kernel; 65-96 x 4096 -> 10240 on the skinny
// kernel in 29-30 us against 37 us (fp32-class) and 32.5 us (fp8 sums) on
// the matrix cores, 128 x 4096 -> 10240 (8 blocks) about even, 65 x 4096 ->
// 14336 (6 blocks) 4-21% slower on it.
int skinny_blocks_per_grid_row(int64_t M) {
  const int64_t blocks = (M + 15) / 16, rows = (blocks + 3) / 4;
  return (int)((blocks + rows - 1) / rows);
}
bool few_tiles_for_matrix_cores(int64_t M, int64_t N) {
  return M <= 256 && N * ((M + 63) / 64) * skinny_blocks_per_grid_row(M) < 81920;
}

// From 17 to 64 rows the skinny kernels serve every block of 16 rows of M
// from one weight step (on wide weights the wide variant, whose workgroups
// load each activation step once for four weight blocks), in time growing
// with N and the number of blocks.  Past 48 rows the matrix-core GEMM's
// 128 x 128 tiles take one round per 2 x CUs tiles, about 44 us for a round
// at K = 4096; the skinny kernel is faster up to N of some 40k (64 x 4096 ->
// 28672: 39 against 44.8 us with fp32-class sums, 39.6-40.2 against 41.7-42.1
// with fp8 sums), the matrix-core GEMM from two rounds on (64 x 4096 ->
// 57344: 64.4 against 69.0 us).
bool wide_enough_for_matrix_cores(int64_t M, int64_t N) { return M > 48 && M <= 64 && N >= 57344; }

// ---- scratch of the no-allocation entry point ----------------------------
// The dynamic quantization's per-block maxima (quant_workspace_bytes(), the
// same for every size) live in this array instead of a caller workspace.
// Each device the library runs on holds its own copy until the process ends.
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address is looked up once per device (hipGetSymbolAddress, with
// that device current) and only that address is handed to kernels.
constexpr size_t kScratchBytes = 4096;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address, looked up on the first call made
// on that device.
fp8_status scratch_for_current_device(const char* fn, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(FP8_ERR_HIP, "%s: hipGetDevice failed: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(FP8_ERR_UNSUPPORTED, "%s: device index %d out of range", fn, dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(FP8_ERR_HIP, "%s: hipGetSymbolAddress(scratch) failed on device %d: %s", fn, dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FP8_OK;
}

// The whole linear: host validation, then the dynamic quantization and the
// scaled GEMM on its codes.  use_scratch: the quantization's per-block
// maxima go to this device's scratch array instead of `workspace`.
fp8_status linear_impl(const char* fn, const uint16_t* x_bf16, int64_t ld_x, const uint8_t* w_q, int64_t ldw,
                       const float* s_w, fp8_scale_mode mode, fp8_accum_mode accum, const uint16_t* bias_bf16,
                       uint8_t* a_q, int64_t ld_aq, float* s_a_out, uint16_t* out_bf16, int64_t ldo, int64_t M,
                       int64_t N, int64_t K, void* workspace, bool use_scratch, hipStream_t stream) {
  if (M < 0 || N < 0) return fail(FP8_ERR_INVALID_ARG, "%s: negative M or N (M=%lld, N=%lld)", fn,
                                  (long long)M, (long long)N);
  if (K < 1) return fail(FP8_ERR_INVALID_ARG, "%s: K must be >= 1 (K=%lld)", fn, (long long)K);
  if (ld_x < K || ld_aq < K || ldw < K) return fail(FP8_ERR_INVALID_ARG, "%s: ld_x/ld_aq/ldw smaller than K", fn);
  if (ldo < N) return fail(FP8_ERR_INVALID_ARG, "%s: ldo smaller than N", fn);
  if (mode != FP8_SCALE_PER_TENSOR && mode != FP8_SCALE_PER_CHANNEL)
    return fail(FP8_ERR_INVALID_ARG, "%s: unknown scale mode %d", fn, (int)mode);
  if (accum != FP8_ACCUM_FP32 && accum != FP8_ACCUM_FP8_MFMA)
    return fail(FP8_ERR_INVALID_ARG, "%s: unknown accumulation mode %d", fn, (int)accum);
  // pointers the problem touches: x and a_q when M > 0, the GEMM's when M and N are
  if (s_a_out == nullptr || (M > 0 && (x_bf16 == nullptr || a_q == nullptr || (!use_scratch && workspace == nullptr))) ||
      (M > 0 && N > 0 && (w_q == nullptr || s_w == nullptr || out_bf16 == nullptr)))
    return fail(FP8_ERR_INVALID_ARG, "%s: null required pointer", fn);
  if (M >= (1ll << 31) || N >= (1ll << 31) || K >= (1ll << 30) || ldw >= (1ll << 40) || ld_aq >= (1ll << 40) ||
      M * ((K + 7) / 8) >= (1ll << 31))
    return fail(FP8_ERR_UNSUPPORTED, "%s: problem too large", fn);
  if (use_scratch) {
    if (fp8w8a8::quant_workspace_bytes() > kScratchBytes)
      return fail(FP8_ERR_UNSUPPORTED, "%s: the quantization needs %zu bytes of scratch, the library holds %zu", fn,
                  fp8w8a8::quant_workspace_bytes(), kScratchBytes);
    fp8_status st = scratch_for_current_device(fn, &workspace);
    if (st != FP8_OK) return st;
  }
  // the quantization, then the GEMM on its codes (nothing to multiply for M == 0 or N == 0)
  fp8_status st = hip_status(fp8w8a8::launch_quant_dynamic(x_bf16, M, K, ld_x, FP8_FORMAT_E4M3, a_q, ld_aq,
                                                           s_a_out, workspace, stream),
                             fn);
  if (st != FP8_OK || M == 0 || N == 0) return st;
  return fp8_scaled_mm_fmt(a_q, ld_aq, FP8_FORMAT_E4M3, w_q, ldw, FP8_FORMAT_E4M3, s_a_out, s_w, mode, accum,
                           bias_bf16, out_bf16, ldo, M, N, K, stream);
}

}  // namespace

extern "C" {

size_t fp8_quant_workspace_bytes(void) { return fp8w8a8::quant_workspace_bytes(); }

const char* fp8_last_error(void) { return g_err; }

fp8_status fp8_quant_dynamic_fmt(const uint16_t* x_bf16, int64_t rows, int64_t cols, int64_t ld_x, fp8_format fmt,
                                 uint8_t* q, int64_t ld_q, float* scale_out, void* workspace, hipStream_t stream) {
  const char* fn = "fp8_quant_dynamic";
  fp8_status st = check_quant(fn, x_bf16, rows, cols, ld_x, q, ld_q);
  if (st == FP8_OK) st = check_fmt(fn, fmt);
  if (st != FP8_OK) return st;
  if (scale_out == nullptr) return fail(FP8_ERR_INVALID_ARG, "%s: null scale_out", fn);
  if (rows > 0 && cols > 0 && workspace == nullptr) return fail(FP8_ERR_INVALID_ARG, "%s: null workspace", fn);
  return hip_status(fp8w8a8::launch_quant_dynamic(x_bf16, rows, cols, ld_x, (int)fmt, q, ld_q, scale_out, workspace,
                                                  stream),
                    fn);
}

fp8_status fp8_quant_dynamic(const uint16_t* x_bf16, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* q_e4m3,
                             int64_t ld_q, float* scale_out, void* workspace, hipStream_t stream) {
  return fp8_quant_dynamic_fmt(x_bf16, rows, cols, ld_x, FP8_FORMAT_E4M3, q_e4m3, ld_q, scale_out, workspace, stream);
}

fp8_status fp8_quant_static_fmt(const uint16_t* x_bf16, int64_t rows, int64_t cols, int64_t ld_x, fp8_format fmt,
                                const float* scale, uint8_t* q, int64_t ld_q, hipStream_t stream) {
  const char* fn = "fp8_quant_static";
  fp8_status st = check_quant(fn, x_bf16, rows, cols, ld_x, q, ld_q);
  if (st == FP8_OK) st = check_fmt(fn, fmt);
  if (st != FP8_OK) return st;
  if (scale == nullptr) return fail(FP8_ERR_INVALID_ARG, "%s: null scale", fn);
  return hip_status(fp8w8a8::launch_quant_static(x_bf16, rows, cols, ld_x, (int)fmt, scale, q, ld_q,
                                                 stream),
                    fn);
}

fp8_status fp8_quant_static(const uint16_t* x_bf16, int64_t rows, int64_t cols, int64_t ld_x, const float* scale,
                            uint8_t* q_e4m3, int64_t ld_q, hipStream_t stream) {
  return fp8_quant_static_fmt(x_bf16, rows, cols, ld_x, FP8_FORMAT_E4M3, scale, q_e4m3, ld_q, stream);
}

fp8_status fp8_quant_dynamic_per_row_fmt(const uint16_t* x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                                         fp8_format fmt, uint8_t* q, int64_t ld_q, float* scales_out, hipStream_t stream) {
  const char* fn = "fp8_quant_dynamic_per_row";
  fp8_status st = check_quant(fn, x_bf16, rows, cols, ld_x, q, ld_q);
  if (st == FP8_OK) st = check_fmt(fn, fmt);
  if (st != FP8_OK) return st;
  if (rows > 0 && scales_out == nullptr) return fail(FP8_ERR_INVALID_ARG, "%s: null scales_out", fn);
  return hip_status(fp8w8a8::launch_quant_per_row(x_bf16, rows, cols, ld_x, (int)fmt, q, ld_q, scales_out,
                                                  stream),
                    fn);
}

fp8_status fp8_quant_dynamic_per_row(const uint16_t* x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                                     uint8_t* q_e4m3, int64_t ld_q, float* scales_out, hipStream_t stream) {
  return fp8_quant_dynamic_per_row_fmt(x_bf16, rows, cols, ld_x, FP8_FORMAT_E4M3, q_e4m3, ld_q, scales_out, stream);
}

size_t fp8_norm_quant_workspace_bytes(int64_t rows) {
  return fp8w8a8::norm_quant_workspace_bytes(rows < 0 ? 0 : rows);
}

fp8_status fp8_add_rmsnorm_quant_dynamic(const uint16_t* h_bf16, int64_t ld_h, const uint16_t* delta_bf16,
                                         int64_t ld_delta, uint16_t* h_out_bf16, int64_t ld_h_out, int64_t rows,
                                         int64_t cols, float eps, uint16_t* y_out_bf16, int64_t ld_y,
                                         uint8_t* q_e4m3, int64_t ld_q, float* scale_out, void* workspace,
                                         hipStream_t stream) {
  const char* fn = "fp8_add_rmsnorm_quant_dynamic";
  fp8_status st = check_quant(fn, h_bf16, rows, cols, ld_h, q_e4m3, ld_q);
  if (st != FP8_OK) return st;
  if (scale_out == nullptr) return fail(FP8_ERR_INVALID_ARG, "%s: null scale_out", fn);
  if (!(eps >= 0.0f) || eps > 3.0e38f) return fail(FP8_ERR_INVALID_ARG, "%s: eps must be finite and >= 0", fn);
  const bool work = rows > 0 && cols > 0;
  if (work && workspace == nullptr) return fail(FP8_ERR_INVALID_ARG, "%s: null workspace", fn);
  if (work && delta_bf16 != nullptr) {
    if (h_out_bf16 == nullptr) return fail(FP8_ERR_INVALID_ARG, "%s: delta given but h_out is null", fn);
    if (ld_delta < cols || ld_h_out < cols)
      return fail(FP8_ERR_INVALID_ARG, "%s: ld_delta/ld_h_out smaller than cols", fn);
  }
  if (work && y_out_bf16 != nullptr && ld_y < cols) return fail(FP8_ERR_INVALID_ARG, "%s: ld_y smaller than cols", fn);
  if (rows >= (1ll << 31)) return fail(FP8_ERR_UNSUPPORTED, "%s: too many rows", fn);
  return hip_status(fp8w8a8::launch_add_rmsnorm_quant(h_bf16, ld_h, delta_bf16, ld_delta, h_out_bf16, ld_h_out, rows,
                                                      cols, eps, y_out_bf16, ld_y, q_e4m3, ld_q, scale_out, workspace,
                                                      stream),
                    fn);
}

fp8_status fp8_silu_mul_quant_dynamic(const uint16_t* gu_bf16, int64_t ld_gu, int64_t rows, int64_t cols,
                                      uint16_t* y_out_bf16, int64_t ld_y, uint8_t* q_e4m3, int64_t ld_q,
                                      float* scale_out, void* workspace, hipStream_t stream) {
  const char* fn = "fp8_silu_mul_quant_dynamic";
  fp8_status st = check_quant(fn, gu_bf16, rows, cols, ld_gu, q_e4m3, ld_q);
  if (st != FP8_OK) return st;
  if (cols > 0 && ld_gu < 2 * cols) return fail(FP8_ERR_INVALID_ARG, "%s: ld_gu smaller than 2 * cols", fn);
  if (scale_out == nullptr) return fail(FP8_ERR_INVALID_ARG, "%s: null scale_out", fn);
  const bool work = rows > 0 && cols > 0;
  if (work && workspace == nullptr) return fail(FP8_ERR_INVALID_ARG, "%s: null workspace", fn);
  if (work && y_out_bf16 != nullptr && ld_y < cols) return fail(FP8_ERR_INVALID_ARG, "%s: ld_y smaller than cols", fn);
  return hip_status(fp8w8a8::launch_silu_mul_quant(gu_bf16, ld_gu, rows, cols, y_out_bf16, ld_y, q_e4m3, ld_q,
                                                   scale_out, workspace, stream),
                    fn);
}

fp8_status fp8_scaled_mm_fmt(const uint8_t* a_q, int64_t lda, fp8_format fmt_a, const uint8_t* w_q, int64_t ldw,
                             fp8_format fmt_w, const float* s_a, const float* s_w, fp8_scale_mode mode,
                             fp8_accum_mode accum, const uint16_t* bias_bf16, uint16_t* out_bf16, int64_t ldo,
                             int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  const char* fn = "fp8_scaled_mm";
  if (check_fmt(fn, fmt_a) != FP8_OK || check_fmt(fn, fmt_w) != FP8_OK) return FP8_ERR_INVALID_ARG;
  if (M < 0 || N < 0) return fail(FP8_ERR_INVALID_ARG, "%s: negative M or N (M=%lld, N=%lld)", fn,
                                  (long long)M, (long long)N);
  if (K < 1) return fail(FP8_ERR_INVALID_ARG, "%s: K must be >= 1 (K=%lld)", fn, (long long)K);
  if (lda < K || ldw < K) return fail(FP8_ERR_INVALID_ARG, "%s: lda/ldw smaller than K", fn);
  if (ldo < N) return fail(FP8_ERR_INVALID_ARG, "%s: ldo smaller than N", fn);
  if (mode != FP8_SCALE_PER_TENSOR && mode != FP8_SCALE_PER_CHANNEL)
    return fail(FP8_ERR_INVALID_ARG, "%s: unknown scale mode %d", fn, (int)mode);
  if (accum != FP8_ACCUM_FP32 && accum != FP8_ACCUM_FP8_MFMA)
    return fail(FP8_ERR_INVALID_ARG, "%s: unknown accumulation mode %d", fn, (int)accum);
  if (a_q == nullptr || w_q == nullptr || s_a == nullptr || s_w == nullptr || out_bf16 == nullptr)
    return fail(FP8_ERR_INVALID_ARG, "%s: null required pointer", fn);
  if (M >= (1ll << 31) || N >= (1ll << 31) || K >= (1ll << 30) || lda >= (1ll << 40) || ldw >= (1ll << 40))
    return fail(FP8_ERR_UNSUPPORTED, "%s: problem too large", fn);
  if (M == 0 || N == 0) return FP8_OK;

  fp8w8a8::GemmArgs g;
  g.a = a_q; g.w = w_q; g.s_a = s_a; g.s_w = s_w; g.bias = bias_bf16; g.out = out_bf16;
  g.lda = lda; g.ldw = ldw; g.ldo = ldo;
  g.M = (int32_t)M; g.N = (int32_t)N; g.K = (int32_t)K;
  g.per_channel = mode == FP8_SCALE_PER_CHANNEL ? 1 : 0;
  g.fmt_a = (int32_t)fmt_a;
  g.fmt_w = (int32_t)fmt_w;
  hipStream_t s = stream;

  const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256);
  const bool fp8_sums = accum == FP8_ACCUM_FP8_MFMA;
  if (((M > 64 && !few_tiles_for_matrix_cores(M, N)) || wide_enough_for_matrix_cores(M, N)) &&
      tiles < (1ll << 31) && fp8w8a8::gemm_mfma_supported(g))
    return hip_status(fp8w8a8::launch_gemm_mfma(g, fp8_sums, s), fn);

  // Skinny kernel, in slices of at most 65535 blocks of 16 rows (grid.y) and
  // 2^25 columns (a launch's threads along x must stay below 2^32: at most
  // 2^21 workgroups of up to 1024 threads).
  const int64_t slice_m = 65535ll * 16, slice_n = 1ll << 25;
  for (int64_t n0 = 0; n0 < N; n0 += slice_n) {
    for (int64_t m0 = 0; m0 < M; m0 += slice_m) {
      fp8w8a8::GemmArgs gs = g;
      gs.a = a_q + m0 * lda;
      gs.w = w_q + n0 * ldw;
      gs.s_w = g.per_channel ? s_w + n0 : s_w;
      gs.bias = bias_bf16 != nullptr ? bias_bf16 + n0 : nullptr;
      gs.out = out_bf16 + m0 * ldo + n0;
      gs.M = (int32_t)((M - m0) < slice_m ? (M - m0) : slice_m);
      gs.N = (int32_t)((N - n0) < slice_n ? (N - n0) : slice_n);
      fp8_status st = hip_status(fp8w8a8::launch_gemm_skinny(gs, s), fn);
      if (st != FP8_OK) return st;
    }
  }
  return FP8_OK;
}

size_t fp8_linear_workspace_bytes(void) { return fp8w8a8::quant_workspace_bytes(); }

fp8_status fp8_linear_dynamic(const uint16_t* x_bf16, int64_t ld_x, const uint8_t* w_q, int64_t ldw,
                              const float* s_w, fp8_scale_mode mode, fp8_accum_mode accum,
                              const uint16_t* bias_bf16, uint8_t* a_q, int64_t ld_aq, float* s_a_out,
                              uint16_t* out_bf16, int64_t ldo, int64_t M, int64_t N, int64_t K, void* workspace,
                              hipStream_t stream) {
  return linear_impl("fp8_linear_dynamic", x_bf16, ld_x, w_q, ldw, s_w, mode, accum, bias_bf16, a_q, ld_aq, s_a_out,
                     out_bf16, ldo, M, N, K, workspace, false, stream);
}

fp8_status fp8_linear_dynamic_noalloc(const uint16_t* x_bf16, int64_t ld_x, const uint8_t* w_q, int64_t ldw,
                                      const float* s_w, fp8_scale_mode mode, fp8_accum_mode accum,
                                      const uint16_t* bias_bf16, uint8_t* a_q, int64_t ld_aq, float* s_a_out,
                                      uint16_t* out_bf16, int64_t ldo, int64_t M, int64_t N, int64_t K,
                                      hipStream_t stream) {
  return linear_impl("fp8_linear_dynamic_noalloc", x_bf16, ld_x, w_q, ldw, s_w, mode, accum, bias_bf16, a_q, ld_aq,
                     s_a_out, out_bf16, ldo, M, N, K, nullptr, true, stream);
}

fp8_status fp8_scaled_mm(const uint8_t* a_q, int64_t lda, const uint8_t* w_q, int64_t ldw, const float* s_a,
                         const float* s_w, fp8_scale_mode mode, const uint16_t* bias_bf16, uint16_t* out_bf16,
                         int64_t ldo, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  return fp8_scaled_mm_fmt(a_q, lda, FP8_FORMAT_E4M3, w_q, ldw, FP8_FORMAT_E4M3, s_a, s_w, mode, FP8_ACCUM_FP32,
                           bias_bf16, out_bf16, ldo, M, N, K, stream);
}

}  // extern "C"
