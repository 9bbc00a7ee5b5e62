// Launchers shared between the C-ABI layer and the kernel translation units.
// Arguments reach these already validated (see api.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fp8w8a8 {

size_t quant_workspace_bytes();

// fmt: 0 = e4m3, 1 = e5m2 (codes written and the scale's denominator).
hipError_t launch_quant_dynamic(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, int fmt, uint8_t* q,
                                int64_t ld_q, float* scale_out, void* workspace, hipStream_t stream);
hipError_t launch_quant_static(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, int fmt,
                               const float* scale, uint8_t* q, int64_t ld_q, hipStream_t stream);
// Fused producers (chained-linears glue) + dynamic per-tensor quantization.
size_t norm_quant_workspace_bytes(int64_t rows);
hipError_t launch_add_rmsnorm_quant(const uint16_t* h, int64_t ld_h, const uint16_t* delta, int64_t ld_delta,
                                    uint16_t* h_out, int64_t ld_h_out, int64_t rows, int64_t cols, float eps,
                                    uint16_t* y_out, int64_t ld_y, uint8_t* q, int64_t ld_q, float* scale_out,
                                    void* workspace, hipStream_t stream);
hipError_t launch_silu_mul_quant(const uint16_t* gu, int64_t ld_gu, int64_t rows, int64_t cols, uint16_t* y_out,
                                 int64_t ld_y, uint8_t* q, int64_t ld_q, float* scale_out, void* workspace,
                                 hipStream_t stream);
hipError_t launch_quant_per_row(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, int fmt, uint8_t* q,
                                int64_t ld_q, float* scales_out, hipStream_t stream);

struct GemmArgs {
  const uint8_t* a;   // [M, K] e4m3fn, pitch lda
  const uint8_t* w;   // [N, K] e4m3fn, pitch ldw
  const float* s_a;   // 1 float
  const float* s_w;   // 1 or N floats
  const uint16_t* bias;  // N bf16 or null
  uint16_t* out;      // [M, N] bf16, pitch ldo
  int64_t lda, ldw, ldo;
  int32_t M, N, K;
  int32_t per_channel;
  int32_t fmt_a, fmt_w;  // 0 = e4m3, 1 = e5m2
};

// Skinny path: any layout; one 16-row block of M per grid row.
hipError_t launch_gemm_skinny(const GemmArgs& g, hipStream_t stream);
// Matrix-core GEMM: requires 16-byte aligned a/w rows and K % 16 == 0.
bool gemm_mfma_supported(const GemmArgs& g);
// fp8_accumulate: fp8 matrix-core sums (fast, 13-bit group sums) instead of
// the exact bf16 path.
hipError_t launch_gemm_mfma(const GemmArgs& g, bool fp8_accumulate, hipStream_t stream);

}  // namespace fp8w8a8
