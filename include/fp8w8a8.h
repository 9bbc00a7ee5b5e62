/*
 * fp8w8a8.h -- C ABI of the MI355X (gfx950) FP8 W8A8 linear layer.
 *
 * The layer, as the pages describe it:
 *   - "Prototype FP8Linear W8A8 runtime quantization" (nm-vllm issue 190),
 *     opening post: weights and activations are quantized at run time to
 *     float8_e4m3fn and multiplied by an FP8 W8A8 GEMM.
 *   - "Fp8 Quantization Support" (compressed-tensors PR 62), description and
 *     recipe: symmetric float quantization (no zero point), one scale per
 *     tensor for weights and input activations.
 *   - "[Kernel] Implement fallback for FP8 channelwise using
 *     torch._scaled_mm" (vLLM PR 6552), description: a per-output-channel
 *     weight scale equals a per-tensor scaled GEMM followed by a rescale of
 *     each output column.  Here that rescale is fused into the GEMM's store.
 *   - "[WIP] FP8 support" (text-generation-inference PR 1484), review
 *     discussion: no 16-alignment restriction, no per-call packing or
 *     padding, and a dedicated path for decode (fewer than 16 rows).
 *
 * Conventions shared by every call:
 *   - Tensor pointers are DEVICE pointers; the caller owns every buffer.
 *     bf16 values travel as their uint16_t bit patterns; e4m3fn values as
 *     uint8_t codes (OCP E4M3, finite-only variant: max 448, 0x7F/0xFF NaN).
 *   - Matrices are row-major with a leading dimension (row pitch) in
 *     elements, ld >= cols.  No alignment is required beyond the element
 *     size; aligned layouts (16-byte rows and base pointers) take faster
 *     paths.  Inputs and outputs must not overlap.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls only
 *     enqueue work: they never allocate, never synchronize and never read
 *     device memory on the host, so they may be captured into a HIP graph.
 *   - Arguments are validated on the host before anything is launched.
 *     A failed validation returns FP8_ERR_INVALID_ARG (or
 *     FP8_ERR_UNSUPPORTED) and launches nothing; a failed launch returns
 *     FP8_ERR_HIP.  fp8_last_error() then returns a text for the calling
 *     thread.  Faults inside a kernel surface at the caller's next
 *     synchronization, as for any HIP kernel.
 *   - Empty problems (rows == 0, cols == 0, M == 0 or N == 0) return
 *     FP8_OK after launching only what is needed to define the outputs
 *     (the quantization calls still write their scale).
 *   - Inputs are expected to be finite.  Non-finite inputs do not fault,
 *     but their codes and outputs are unspecified.
 */
#ifndef FP8W8A8_H
#define FP8W8A8_H

#include <stddef.h>
#include <stdint.h>

/* The HIP stream type, declared exactly as the HIP runtime declares it, so
 * this header needs no HIP include (a repeated identical typedef is valid
 * C11 and C++). */
typedef struct ihipStream_t* hipStream_t;

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FP8_OK = 0,
  FP8_ERR_INVALID_ARG = 1,
  FP8_ERR_UNSUPPORTED = 2,
  FP8_ERR_HIP = 3
} fp8_status;

typedef enum {
  FP8_SCALE_PER_TENSOR = 0,  /* s_w holds 1 float, used for every column */
  FP8_SCALE_PER_CHANNEL = 1  /* s_w holds N floats, s_w[n] for column n  */
} fp8_scale_mode;

/*
 * How fp8_scaled_mm_fmt and fp8_linear_dynamic sum the products (each
 * product of two e4m3 values is exact in every mode; fp8_scaled_mm always
 * sums as FP8_ACCUM_FP32).
 *   FP8_ACCUM_FP32      sums with fp32-class precision: the codes are
 *                       converted to bf16 in registers (exact) and run on the
 *                       bf16 matrix cores.  The default.
 *   FP8_ACCUM_FP8_MFMA  the fp8 matrix cores (v_mfma_f32_32x32x64_f8f6f4),
 *                       twice the bf16 rate, where the matrix-core GEMM runs
 *                       (see fp8_scaled_mm).  On gfx950 they sum each group
 *                       of 8 products keeping 13 bits below the group's
 *                       largest product, so small products next to large
 *                       ones are truncated.  Where the call runs the skinny
 *                       kernel (most M <= 64, small problems up to 256 rows,
 *                       and layouts the matrix-core GEMM does not take), it
 *                       sums with the FP32 path in either mode.
 */
typedef enum {
  FP8_ACCUM_FP32 = 0,
  FP8_ACCUM_FP8_MFMA = 1
} fp8_accum_mode;

/* Largest e4m3fn magnitude; the dynamic scale maps amax onto it. */
#define FP8_E4M3_MAX 448.0f

/*
 * Bytes of device workspace fp8_quant_dynamic needs (a few KiB).  The
 * workspace needs no initialization; its contents are scratch between the
 * kernels of one call, so calls that run concurrently on different streams
 * need different workspaces.
 */
size_t fp8_quant_workspace_bytes(void);

/*
 * Dynamic per-tensor quantization of bf16 activations
 * ("Prototype FP8Linear W8A8 runtime quantization", opening post: the
 * activation scale is computed per call from the live tensor).
 *
 *   amax      = max |x| over all rows x cols elements (exact)
 *   *scale_out = amax / 448 rounded once to float32; 1.0 when amax == 0
 *   q[r, c]   = e4m3fn(x[r, c] / scale) -- a correctly rounded float32
 *               division, then round-to-nearest-even with saturation to
 *               +-448; the sign of zero is kept.
 *
 *   x_bf16   [rows, cols], row pitch ld_x >= cols      (input)
 *   q_e4m3   [rows, cols], row pitch ld_q >= cols      (output)
 *   scale_out 1 float in device memory                 (output, never read back)
 *   workspace fp8_quant_workspace_bytes() bytes         (scratch)
 * Errors: INVALID_ARG for null x/q/scale_out/workspace (when rows*cols > 0;
 * scale_out is always required), negative sizes, or ld < cols.
 */
fp8_status fp8_quant_dynamic(const uint16_t* x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                             uint8_t* q_e4m3, int64_t ld_q, float* scale_out,
                             void* workspace, hipStream_t stream);

/*
 * Quantization with a given per-tensor scale (a calibrated, static
 * activation scale as in the "Fp8 Quantization Support" recipe, where the
 * input activations get one scale per tensor).  q = e4m3fn(x / *scale), with
 * the same division, rounding and saturation as fp8_quant_dynamic.  Values
 * beyond 448 * scale saturate to +-448.
 *   scale  1 float in device memory, finite and > 0   (input)
 * Errors: as fp8_quant_dynamic (no workspace).
 */
fp8_status fp8_quant_static(const uint16_t* x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                            const float* scale, uint8_t* q_e4m3, int64_t ld_q, hipStream_t stream);

/*
 * Per-row dynamic quantization: row r gets its own scale from its own amax
 * (the channelwise weight scale of "[Kernel] Implement fallback for FP8
 * channelwise using torch._scaled_mm": weight row n is output channel n).
 * Used to quantize an nn.Linear weight [N, K] on the device at load time.
 *   scales_out  rows floats in device memory (output); an all-zero row
 *               gets scale 1.0.
 * Errors: as fp8_quant_dynamic (no workspace).
 */
fp8_status fp8_quant_dynamic_per_row(const uint16_t* x_bf16, int64_t rows, int64_t cols,
                                     int64_t ld_x, uint8_t* q_e4m3, int64_t ld_q,
                                     float* scales_out, hipStream_t stream);

/*
 * Scaled FP8 GEMM with the rescale epilogue fused into the store.
 *
 * Defined by "Prototype FP8Linear W8A8 runtime quantization" (opening post:
 * an FP8 W8A8 linear multiplies e4m3fn activations by e4m3fn weights, each
 * with its own scale) and "[Kernel] Implement fallback for FP8 channelwise
 * using torch._scaled_mm" (description: a per-output-channel weight scale is
 * a per-tensor scaled GEMM followed by a rescale of each output column;
 * s_w[n] does not depend on k, so the rescale factors out of the k-sum and is
 * applied once per output element, here in the GEMM's store):
 *
 *   out[m, n] = bf16_rne( (sum_k dec(a_q[m, k]) * dec(w_q[n, k]))
 *                         * (s_a[0] * s_w[n or 0]) + bias[n] )
 *
 * Products of two e4m3 values are exact and are summed with fp32-class
 * precision (FP8_ACCUM_FP32 below); the scale product s_a * s_w is formed in
 * float32 and applied with one fused multiply-add together with the bias.
 * Per-channel with all s_w[n] equal gives bit-identical output to
 * per-tensor with that value.
 *
 *   a_q    [M, K] e4m3fn, row pitch lda >= K          (activations)
 *   w_q    [N, K] e4m3fn, row pitch ldw >= K          (nn.Linear weight;
 *                                                      out = A * W^T)
 *   s_a    1 float (device)                            (activation scale)
 *   s_w    1 float (PER_TENSOR) or N floats (PER_CHANNEL) (device)
 *   bias   N bf16 values (device), or NULL for none
 *   out    [M, N] bf16, row pitch ldo >= N            (output)
 * Kernels: the skinny (decode) kernel streams the weight once for up to 64
 * rows of M (one workgroup serves all of them; on wide weights, with M from
 * 17, each workgroup also loads every activation step once for four weight
 * blocks), with no padding or repacking; the LDS-staged matrix-core GEMM
 * runs 256 x 256 tiles, or 128 x 128 tiles where the larger ones are too
 * few to occupy the GPU.
 * M <= 64 runs the skinny kernel, but for 48 < M <= 64 with N >= 57344.
 * Larger M runs the matrix-core GEMM, but for problems too small for its
 * tiles: M <= 256 and N * R * B below 81920, where the skinny kernel runs
 * R = ceil(M / 64) grid rows of B = ceil(ceil(M / 16) / R) blocks of 16
 * rows.  Layouts the matrix-core GEMM does not take (rows not 16-byte
 * aligned or K % 16 != 0) run the skinny kernel, which then reads the weight
 * once per grid row of up to 64 rows of M (per 16 rows for unaligned
 * layouts).  Any M, N, K >= 1 is accepted.
 * Errors: INVALID_ARG for null pointers (bias may be NULL), negative M or
 * N, K < 1, lda/ldw < K, ldo < N, or an unknown scale mode; UNSUPPORTED for
 * M or N >= 2^31, K >= 2^30 or pitches >= 2^40.  M == 0 or N == 0 is an
 * OK no-op.
 */
fp8_status fp8_scaled_mm(const uint8_t* a_q, int64_t lda, const uint8_t* w_q, int64_t ldw,
                         const float* s_a, const float* s_w, fp8_scale_mode mode,
                         const uint16_t* bias_bf16, uint16_t* out_bf16, int64_t ldo,
                         int64_t M, int64_t N, int64_t K, hipStream_t stream);

/*
 * The whole W8A8 linear in one call: dynamic per-tensor quantization of the
 * bf16 activations (exactly fp8_quant_dynamic: s_a = amax / 448, codes into
 * a_q) followed by fp8_scaled_mm on those codes with that scale ("Prototype
 * FP8Linear W8A8 runtime quantization", opening post: both steps run at
 * every call).  Outputs are bit-identical to making the two calls.
 *
 *   x      [M, K] bf16, row pitch ld_x >= K           (activations, input)
 *   w_q, ldw, s_w, mode, accum, bias, out, ldo        as in fp8_scaled_mm
 *   a_q    [M, K] e4m3fn, row pitch ld_aq >= K        (codes, output)
 *   s_a_out 1 float                                    (scale, output)
 *   workspace  fp8_linear_workspace_bytes() of device memory, no
 *          initialization needed (scratch of the quantization, as for
 *          fp8_quant_dynamic).
 * Errors: INVALID_ARG for a null s_a_out, a null x, a_q or workspace with
 * M > 0, a null w_q, s_w or out with M > 0 and N > 0 (bias may always be
 * NULL), negative M or N, K < 1, a pitch below its minimum, or an unknown
 * scale or accumulation mode; UNSUPPORTED for sizes past the limits of
 * fp8_quant_dynamic and fp8_scaled_mm.
 */
size_t fp8_linear_workspace_bytes(void);
fp8_status fp8_linear_dynamic(const uint16_t* x_bf16, int64_t ld_x, const uint8_t* w_q, int64_t ldw,
                              const float* s_w, fp8_scale_mode mode, fp8_accum_mode accum,
                              const uint16_t* bias_bf16, uint8_t* a_q, int64_t ld_aq, float* s_a_out,
                              uint16_t* out_bf16, int64_t ldo, int64_t M, int64_t N, int64_t K,
                              void* workspace, hipStream_t stream);

/*
 * fp8_linear_dynamic for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops and harnesses that forbid
 * allocation.  The arguments and results are fp8_linear_dynamic's without
 * the workspace: the quantization's scratch (4 KiB of per-block maxima,
 * the same for every problem size) is a fixed array inside the library,
 * one per device, held until the process ends.  The call allocates
 * nothing; its first call on a device looks up that device's array.
 * Every call on a device shares that array, so calls that overlap on one
 * device (concurrent streams, or threads) race and must be serialized by
 * the caller; nothing in it needs to start at zero.
 * Errors: as fp8_linear_dynamic (no workspace argument to check);
 * FP8_ERR_HIP if the array's address cannot be looked up.
 */
fp8_status fp8_linear_dynamic_noalloc(const uint16_t* x_bf16, int64_t ld_x, const uint8_t* w_q, int64_t ldw,
                                      const float* s_w, fp8_scale_mode mode, fp8_accum_mode accum,
                                      const uint16_t* bias_bf16, uint8_t* a_q, int64_t ld_aq, float* s_a_out,
                                      uint16_t* out_bf16, int64_t ldo, int64_t M, int64_t N, int64_t K,
                                      hipStream_t stream);

/*
 * Producer-fused quantization: the step that feeds a linear, computed and
 * quantized in the same pass, so its bf16 result never travels through
 * memory.  The review of "[WIP] FP8 support" (text-generation-inference PR
 * 1484) asks to remove the unnecessary operations around the FP8 GEMM; the
 * pages do not define the producers themselves, so their definitions are
 * readings: a Llama-shaped block's residual add, unit-weight RMS
 * normalization, and gate-first SiLU*mul, each rounded once to bf16.
 * The quantization is exactly fp8_quant_dynamic's, applied to those bf16
 * values.  Workspace contents are scratch between the kernels of one call.
 */

/* Bytes of workspace fp8_add_rmsnorm_quant_dynamic needs for `rows` rows. */
size_t fp8_norm_quant_workspace_bytes(int64_t rows);

/*
 * h' = bf16(h + delta)             (float32 add, one rounding; skipped when
 *                                   delta is NULL: h' = h)
 * y  = bf16(h' / sqrt(mean_c(h'^2) + eps))   per row, float64 math, one
 *                                             rounding to bf16
 * (q, *scale_out) = dynamic per-tensor quantization of y
 *
 *   h_bf16     [rows, cols], pitch ld_h                 (residual stream in)
 *   delta_bf16 [rows, cols], pitch ld_delta, or NULL    (added first)
 *   h_out_bf16 [rows, cols], pitch ld_h_out: receives h' (required iff
 *              delta is given; must not overlap h or delta)
 *   eps        finite, >= 0 (1e-5 for Llama-shaped blocks)
 *   y_out_bf16 [rows, cols], pitch ld_y, or NULL: receives y, the exact
 *              values that were quantized
 *   q_e4m3, ld_q, scale_out  as fp8_quant_dynamic
 *   workspace  fp8_norm_quant_workspace_bytes(rows) bytes
 * Errors: as fp8_quant_dynamic, plus INVALID_ARG for a missing h_out when
 * delta is given, pitches smaller than cols, or a negative/non-finite eps.
 */
fp8_status fp8_add_rmsnorm_quant_dynamic(const uint16_t* h_bf16, int64_t ld_h,
                                         const uint16_t* delta_bf16, int64_t ld_delta,
                                         uint16_t* h_out_bf16, int64_t ld_h_out,
                                         int64_t rows, int64_t cols, float eps,
                                         uint16_t* y_out_bf16, int64_t ld_y,
                                         uint8_t* q_e4m3, int64_t ld_q, float* scale_out,
                                         void* workspace, hipStream_t stream);

/*
 * m = bf16(silu(g) * u), silu(g) = g / (1 + exp(-g)) in float64, where row r
 * of gu_bf16 holds the gate in columns [0, cols) and the up projection in
 * [cols, 2 cols) (a fused gate_up linear's output);
 * (q, *scale_out) = dynamic per-tensor quantization of m.
 *
 *   gu_bf16   [rows, 2 cols], pitch ld_gu >= 2 cols     (input)
 *   y_out_bf16 [rows, cols], pitch ld_y, or NULL: receives m
 *   q_e4m3    [rows, cols], pitch ld_q; scale_out as fp8_quant_dynamic
 *   workspace fp8_quant_workspace_bytes() bytes
 * Errors: as fp8_quant_dynamic, plus INVALID_ARG for ld_gu < 2 cols.
 */
fp8_status fp8_silu_mul_quant_dynamic(const uint16_t* gu_bf16, int64_t ld_gu, int64_t rows,
                                      int64_t cols, uint16_t* y_out_bf16, int64_t ld_y,
                                      uint8_t* q_e4m3, int64_t ld_q, float* scale_out,
                                      void* workspace, hipStream_t stream);

/*
 * fp8 formats.  E4M3 is the pages' float8_e4m3fn (max 448) and the format of
 * every call above.  E5M2 is OCP float8_e5m2 (max 57344; 2 mantissa bits,
 * wider range), the extension the "Fp8 Quantization Support"
 * (compressed-tensors PR 62) description names for the same quantization
 * scheme.  The *_fmt calls below are the calls above with the format of
 * each fp8 tensor as an argument: the same scale rule (amax / max of the
 * format), division, round-to-nearest-even and saturation (to +-max);
 * e5m2 infinities and NaNs are never produced from finite inputs.
 */
typedef enum { FP8_FORMAT_E4M3 = 0, FP8_FORMAT_E5M2 = 1 } fp8_format;

fp8_status fp8_quant_dynamic_fmt(const uint16_t* x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                                 fp8_format fmt, uint8_t* q, int64_t ld_q, float* scale_out,
                                 void* workspace, hipStream_t stream);
fp8_status fp8_quant_static_fmt(const uint16_t* x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                                fp8_format fmt, const float* scale, uint8_t* q, int64_t ld_q,
                                hipStream_t stream);
fp8_status fp8_quant_dynamic_per_row_fmt(const uint16_t* x_bf16, int64_t rows, int64_t cols,
                                         int64_t ld_x, fp8_format fmt, uint8_t* q, int64_t ld_q,
                                         float* scales_out, hipStream_t stream);
/*
 * fp8_scaled_mm with the format of each operand and the accumulation mode
 * as arguments: a_q holds fmt_a codes, w_q fmt_w codes (any mix), and
 * `accum` selects how products are summed (see fp8_accum_mode;
 * FP8_ACCUM_FP32 gives exactly fp8_scaled_mm).  Otherwise, and for its
 * errors (plus INVALID_ARG for an unknown format or accumulation mode), as
 * fp8_scaled_mm.
 */
fp8_status fp8_scaled_mm_fmt(const uint8_t* a_q, int64_t lda, fp8_format fmt_a,
                             const uint8_t* w_q, int64_t ldw, fp8_format fmt_w,
                             const float* s_a, const float* s_w, fp8_scale_mode mode,
                             fp8_accum_mode accum, const uint16_t* bias_bf16, uint16_t* out_bf16,
                             int64_t ldo, int64_t M, int64_t N, int64_t K, hipStream_t stream);

/* Text describing the calling thread's most recent non-OK status. */
const char* fp8_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8W8A8_H */
