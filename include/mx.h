/*
 * mx.h -- C ABI of the gfx950 microscaling library: per-32 activation quantization to
 * E4M3 + E8M0 and block-scaled GEMMs over E4M3 / E2M1 operands.
 *
 * Formats (the "formats.py" page, module docstring and FP4_TABLE; the "hip_quant PKG-INFO"
 * page, FP8 Formats table and native MXFP4 section):
 *   E4M3  one byte per value, e4m3fn: 1 sign, 4 exponent (bias 7), 3 mantissa bits, no
 *         infinities, 0x7F / 0xFF are NaN, largest finite 448, subnormals m * 2^-9.
 *   E2M1  4 bits per value, two per byte: byte j of a row holds element 2j in its LOW nibble
 *         and element 2j+1 in its HIGH nibble; code -> {0,.5,1,1.5,2,3,4,6}, bit 3 = sign.
 *   E8M0  one byte b per scale, value 2^(b-127); 255 is NaN.
 *   bf16  raw 16-bit patterns (the top half of an fp32).
 *
 * Conventions shared by every entry point
 *   - All buffers are device memory owned by the caller; the library never allocates, frees or
 *     synchronizes.  Work is enqueued on `stream` (a hipStream_t; NULL = the null stream).
 *   - Row-major, contiguous rows.  GEMMs are "NT": C[M,N] = A[M,K] . B[N,K]^T, both operands
 *     K-major (the layout the "hip_quant PKG-INFO" page states for its FP8 linear and its
 *     native MXFP4 call).
 *   - K must be a positive multiple of 32 (one scale per 32 consecutive K; the "formats.py"
 *     act_scale refuses other K).  M, N and batch may be any value >= 0; when M, N or batch is 0
 *     the call returns MX_OK and enqueues nothing.
 *   - The code / packed operand base pointers (x, q, a, b) must be 16-byte aligned; scale,
 *     bias and output pointers need no alignment.  Batch strides of the 16-byte-aligned
 *     operands must keep every batch 16-byte aligned.
 *   - Strides are counted in elements of each buffer: bytes for code, packed and scale buffers,
 *     bf16 elements for c, x and bias.  A stride of 0 broadcasts one input to every batch; an
 *     output stride of 0 with batch > 1 is refused.
 *   - Each matrix (one batch) must hold fewer than 2^31 elements; batch <= 65535.
 *   - Argument errors are returned before any HIP call.  A launch failure is reported as
 *     MX_ERR_LAUNCH; faults inside a kernel surface at the caller's next synchronization.
 *   - Inputs the formats refuse are outside the contract and are NOT checked on the device:
 *     NaN E4M3 codes, scale byte 255, non-finite activations.  Their outputs are unspecified.
 *   - All entry points are thread-safe and stateless apart from a per-device capability cache and,
 *     per kernel and device, the one-time raise of its dynamic LDS limit on first launch.
 */
#ifndef MX_H_
#define MX_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  MX_OK = 0,
  MX_ERR_NULL = -1,    /* a required pointer is NULL (or caps == NULL)                       */
  MX_ERR_SHAPE = -2,   /* K not a positive multiple of 32, a negative size, too large a size */
  MX_ERR_ALIGN = -3,   /* an operand base or batch stride breaks 16-byte alignment           */
  MX_ERR_STRIDE = -4,  /* negative stride, or output stride 0 with batch > 1                 */
  MX_ERR_DEVICE = -5,  /* no HIP device, or the current device is not gfx950                 */
  MX_ERR_LAUNCH = -6,  /* the kernel launch itself failed                                    */
  MX_ERR_WORKSPACE = -7 /* split-K workspace NULL, smaller than asked or not 256-B aligned    */
};

typedef struct mx_caps {
  int32_t available;      /* 1 when the current device is gfx950 and the kernels can run     */
  int32_t device;         /* current HIP device ordinal, -1 when there is none               */
  int32_t compute_units;  /* CUs of the current device, 0 when there is none                 */
  int32_t reserved;
  char arch[64];          /* gcnArchName of the current device, "" when there is none         */
  char reason[128];       /* why `available` is 0, "" otherwise                               */
} mx_caps;

/* Fills *caps for the calling thread's current device.  Safe to call without any GPU (the
 * "hip_quant PKG-INFO" page's native MXFP4 section asks the same of its capability query).
 * Returns MX_OK when the kernels can run, MX_ERR_DEVICE when they cannot, MX_ERR_NULL when
 * caps is NULL. */
int mx_capability(mx_caps* caps);

/* Static English text for a status code (never NULL). */
const char* mx_status_str(int status);

/* ---------------------------------------------------------------------------------------------
 * act_quant -- the "formats.py" page, act_scale + act_quant (with _log2_ceil_pow2), per 32
 * consecutive elements of each row:
 *   amax = max(max |x|, fp32(1e-4))                        in fp32
 *   E    = ceil(log2(fp32(amax * fp32(1/448))))             from the fp32 exponent bits
 *   q    = e4m3_rne(clamp(x * 2^-E, -448, 448))              round to nearest even
 * x  : bf16 [M, K]           (16-byte aligned)
 * q  : E4M3 codes [M, K]     (16-byte aligned; written)
 * s  : E8M0 bytes [M, K/32]  (the byte E + 127; written)
 * The result is bit-exact: every code and scale byte is defined by the steps above.
 * ------------------------------------------------------------------------------------------- */
int mx_act_quant(const void* x, void* q, void* s, int64_t M, int64_t K, void* stream);

/* `batch` independent [M, K] problems; batch i reads x + i*stride_x (bf16 elements) and writes
 * q + i*stride_q and s + i*stride_s (bytes).  stride_q and stride_s must not be 0 when
 * batch > 1. */
int mx_act_quant_strided_batched(const void* x, void* q, void* s, int64_t M, int64_t K,
                                 int64_t batch, int64_t stride_x, int64_t stride_q,
                                 int64_t stride_s, void* stream);

/* ---------------------------------------------------------------------------------------------
 * act_quant_fp4 -- the MXFP4 activation producer (packed E2M1 + per-32 E8M0), the operand format
 * of the "formats.py" page (FP4_TABLE, low nibble first, one E8M0 byte per 32 values) and of the
 * "hip_quant PKG-INFO" page's native MXFP4 call.  The pages give no producer rule; this one is
 * act_quant's with E2M1's largest magnitude 6 in place of 448, per 32 consecutive elements:
 *   amax = max(max |x|, fp32(1e-4))
 *   E    = ceil(log2(amax / 6)), exactly (the smallest E with amax <= 6 * 2^E)
 *   code = E2M1 value nearest x * 2^-E, ties to the even code, sign kept (nothing is clipped)
 * x  : bf16 [M, K]                (16-byte aligned)
 * q  : packed E2M1 [M, K/2]       (16-byte aligned; written; element 2j in the low nibble)
 * s  : E8M0 bytes [M, K/32]       (written)
 * Bit-exact.  The batched form: batch i at x + i*stride_x, q + i*stride_q, s + i*stride_s.
 * ------------------------------------------------------------------------------------------- */
int mx_act_quant_fp4(const void* x, void* q, void* s, int64_t M, int64_t K, void* stream);
int mx_act_quant_fp4_strided_batched(const void* x, void* q, void* s, int64_t M, int64_t K,
                                     int64_t batch, int64_t stride_x, int64_t stride_q,
                                     int64_t stride_s, void* stream);

/* ---------------------------------------------------------------------------------------------
 * Block-scaled GEMM: C[m,n] = bf16_rne( sum_k A[m,k] B[n,k] + bias[n] ), the sum accumulated
 * in fp32 on the matrix cores, the bias (when given) added in fp32 before the one bf16
 * rounding (the "AstrAI commit log" page, fused-bias commit).  Decoded operands:
 *   A[m,k] = e4m3(a[m,k]) * 2^(a_scale[m, k/32] - 127)                    (fp8 A)
 *   A[m,k] = e2m1(nibble k of a[m, :]) * 2^(a_scale[m, k/32] - 127)       (fp4 A)
 *   B[n,k] = e2m1(nibble k of b[n, :]) * 2^(b_scale[n, k/32] - 127)       (fp4 B, MXFP4)
 *   B[n,k] = e4m3(b[n,k]) * 2^(b_scale[n/32, k/32] - 127)                 (fp8 B, 32x32 blocks)
 * ("formats.py": decode_fp4, decode_fp8_block; act_qdq for the activation side.)
 * Buffers:
 *   a       fp8: [M, K] bytes;  fp4: [M, K/2] bytes           (16-byte aligned)
 *   a_scale [M, K/32] bytes
 *   b       fp4: [N, K/2] bytes; fp8: [N, K] bytes            (16-byte aligned)
 *   b_scale fp4: [N, K/32] bytes; fp8: [ceil(N/32), K/32] bytes
 *   bias    bf16 [N]   (the _bias variants only; must not be NULL there)
 *   c       bf16 [M, N] (written)
 * Accuracy: each output satisfies |c - ref| <= 2^-7 |ref| + 2^-20 sum_k |A[m,k] B[n,k]|
 * against the exact ref = sum_k A B + bias, for inputs whose scaled products stay within fp32
 * range.
 * ------------------------------------------------------------------------------------------- */
int mx_gemm_fp8_fp4(const void* a, const void* a_scale, const void* b, const void* b_scale,
                    void* c, int64_t M, int64_t N, int64_t K, void* stream);
int mx_gemm_fp8_fp4_bias(const void* a, const void* a_scale, const void* b, const void* b_scale,
                         const void* bias, void* c, int64_t M, int64_t N, int64_t K,
                         void* stream);
int mx_gemm_fp8_fp4_strided_batched(const void* a, const void* a_scale, const void* b,
                                    const void* b_scale, void* c, int64_t M, int64_t N, int64_t K,
                                    int64_t batch, int64_t stride_a, int64_t stride_a_scale,
                                    int64_t stride_b, int64_t stride_b_scale, int64_t stride_c,
                                    void* stream);
int mx_gemm_fp8_fp4_bias_strided_batched(const void* a, const void* a_scale, const void* b,
                                         const void* b_scale, const void* bias, void* c,
                                         int64_t M, int64_t N, int64_t K, int64_t batch,
                                         int64_t stride_a, int64_t stride_a_scale,
                                         int64_t stride_b, int64_t stride_b_scale,
                                         int64_t stride_bias, int64_t stride_c, void* stream);

int mx_gemm_fp8_fp8(const void* a, const void* a_scale, const void* b, const void* b_scale,
                    void* c, int64_t M, int64_t N, int64_t K, void* stream);
int mx_gemm_fp8_fp8_bias(const void* a, const void* a_scale, const void* b, const void* b_scale,
                         const void* bias, void* c, int64_t M, int64_t N, int64_t K,
                         void* stream);
int mx_gemm_fp8_fp8_strided_batched(const void* a, const void* a_scale, const void* b,
                                    const void* b_scale, void* c, int64_t M, int64_t N, int64_t K,
                                    int64_t batch, int64_t stride_a, int64_t stride_a_scale,
                                    int64_t stride_b, int64_t stride_b_scale, int64_t stride_c,
                                    void* stream);
int mx_gemm_fp8_fp8_bias_strided_batched(const void* a, const void* a_scale, const void* b,
                                         const void* b_scale, const void* bias, void* c,
                                         int64_t M, int64_t N, int64_t K, int64_t batch,
                                         int64_t stride_a, int64_t stride_a_scale,
                                         int64_t stride_b, int64_t stride_b_scale,
                                         int64_t stride_bias, int64_t stride_c, void* stream);

/* Both operands MXFP4 (E2M1 + per-row-32 E8M0), as the skinny A4W4 shapes of the
 * "fp4-gemm README" page (release-gate shapes) need. */
int mx_gemm_fp4_fp4(const void* a, const void* a_scale, const void* b, const void* b_scale,
                    void* c, int64_t M, int64_t N, int64_t K, void* stream);
int mx_gemm_fp4_fp4_bias(const void* a, const void* a_scale, const void* b, const void* b_scale,
                         const void* bias, void* c, int64_t M, int64_t N, int64_t K,
                         void* stream);
int mx_gemm_fp4_fp4_strided_batched(const void* a, const void* a_scale, const void* b,
                                    const void* b_scale, void* c, int64_t M, int64_t N, int64_t K,
                                    int64_t batch, int64_t stride_a, int64_t stride_a_scale,
                                    int64_t stride_b, int64_t stride_b_scale, int64_t stride_c,
                                    void* stream);
int mx_gemm_fp4_fp4_bias_strided_batched(const void* a, const void* a_scale, const void* b,
                                         const void* b_scale, const void* bias, void* c,
                                         int64_t M, int64_t N, int64_t K, int64_t batch,
                                         int64_t stride_a, int64_t stride_a_scale,
                                         int64_t stride_b, int64_t stride_b_scale,
                                         int64_t stride_bias, int64_t stride_c, void* stream);

/* ---------------------------------------------------------------------------------------------
 * GEMM with a quantized output: the next layer's activation operand instead of bf16.
 *
 * The "fp4-gemm README" page lists an epilogue that emits the following projection's quantized
 * input directly, so that no bf16 tensor is materialized and no separate quantization launch is
 * needed (API list and the paragraph after the schedule variants); the "AstrAI commit log" page
 * has an FP8-in / FP8-out GEMM op.  Here the output format is this library's activation format:
 *   y[m,n]  = bf16_rne( sum_k A[m,k] B[n,k] + bias[n] )     exactly the value the bf16 entry
 *                                                           points above write for the same call;
 *   (q, q_scale) = act_quant(y)                             per 32 consecutive n of each row,
 *                                                           exactly as mx_act_quant does.
 * The result is byte-identical to mx_gemm_* followed by mx_act_quant on the bf16 output.
 * mx_gemm_fp4_fp4_quant writes the A4W4 layer's next operand instead: packed E2M1 (q [M, N/2],
 * low nibble first) + E8M0 from mx_act_quant_fp4 of the bf16 output, byte-identical to
 * mx_gemm_fp4_fp4 followed by mx_act_quant_fp4.
 * The _bias_gelu_quant forms apply GELU (as mx_gemm_*_bias_gelu does) before the bf16 rounding
 * that is quantized, like the "fp4-gemm README" page's bias + GELU epilogue that emits packed
 * FP4; they equal mx_gemm_*_bias_gelu followed by the producer of the kind's format.
 *   bias     bf16 [N], or NULL for no bias
 *   q        E4M3 codes [M, N] (E2M1 kind: packed [M, N/2]) (16-byte aligned; written)
 *   q_scale  E8M0 bytes [M, N/32] (written)
 * N must be a multiple of 32 (MX_ERR_SHAPE otherwise).  Operands, formats and the other rules as
 * for mx_gemm_fp8_fp4 / mx_gemm_fp8_fp8.  Batched: q + i*stride_q, q_scale + i*stride_q_scale
 * (bytes; stride_q a multiple of 16; neither 0 when batch > 1).
 * ------------------------------------------------------------------------------------------- */
int mx_gemm_fp8_fp4_quant(const void* a, const void* a_scale, const void* b, const void* b_scale,
                          const void* bias, void* q, void* q_scale, int64_t M, int64_t N,
                          int64_t K, void* stream);
int mx_gemm_fp8_fp4_quant_strided_batched(const void* a, const void* a_scale, const void* b,
                                          const void* b_scale, const void* bias, void* q,
                                          void* q_scale, int64_t M, int64_t N, int64_t K,
                                          int64_t batch, int64_t stride_a, int64_t stride_a_scale,
                                          int64_t stride_b, int64_t stride_b_scale,
                                          int64_t stride_bias, int64_t stride_q,
                                          int64_t stride_q_scale, void* stream);
int mx_gemm_fp8_fp8_quant(const void* a, const void* a_scale, const void* b, const void* b_scale,
                          const void* bias, void* q, void* q_scale, int64_t M, int64_t N,
                          int64_t K, void* stream);
int mx_gemm_fp8_fp8_quant_strided_batched(const void* a, const void* a_scale, const void* b,
                                          const void* b_scale, const void* bias, void* q,
                                          void* q_scale, int64_t M, int64_t N, int64_t K,
                                          int64_t batch, int64_t stride_a, int64_t stride_a_scale,
                                          int64_t stride_b, int64_t stride_b_scale,
                                          int64_t stride_bias, int64_t stride_q,
                                          int64_t stride_q_scale, void* stream);
int mx_gemm_fp4_fp4_quant(const void* a, const void* a_scale, const void* b, const void* b_scale,
                          const void* bias, void* q, void* q_scale, int64_t M, int64_t N,
                          int64_t K, void* stream);
int mx_gemm_fp4_fp4_quant_strided_batched(const void* a, const void* a_scale, const void* b,
                                          const void* b_scale, const void* bias, void* q,
                                          void* q_scale, int64_t M, int64_t N, int64_t K,
                                          int64_t batch, int64_t stride_a, int64_t stride_a_scale,
                                          int64_t stride_b, int64_t stride_b_scale,
                                          int64_t stride_bias, int64_t stride_q,
                                          int64_t stride_q_scale, void* stream);
int mx_gemm_fp8_fp4_bias_gelu_quant(const void* a, const void* a_scale, const void* b,
                                    const void* b_scale, const void* bias, void* q, void* q_scale,
                                    int64_t M, int64_t N, int64_t K, void* stream);
int mx_gemm_fp8_fp4_bias_gelu_quant_strided_batched(const void* a, const void* a_scale,
                                                    const void* b, const void* b_scale,
                                                    const void* bias, void* q, void* q_scale,
                                                    int64_t M, int64_t N, int64_t K, int64_t batch,
                                                    int64_t stride_a, int64_t stride_a_scale,
                                                    int64_t stride_b, int64_t stride_b_scale,
                                                    int64_t stride_bias, int64_t stride_q,
                                                    int64_t stride_q_scale, void* stream);
int mx_gemm_fp8_fp8_bias_gelu_quant(const void* a, const void* a_scale, const void* b,
                                    const void* b_scale, const void* bias, void* q, void* q_scale,
                                    int64_t M, int64_t N, int64_t K, void* stream);
int mx_gemm_fp8_fp8_bias_gelu_quant_strided_batched(const void* a, const void* a_scale,
                                                    const void* b, const void* b_scale,
                                                    const void* bias, void* q, void* q_scale,
                                                    int64_t M, int64_t N, int64_t K, int64_t batch,
                                                    int64_t stride_a, int64_t stride_a_scale,
                                                    int64_t stride_b, int64_t stride_b_scale,
                                                    int64_t stride_bias, int64_t stride_q,
                                                    int64_t stride_q_scale, void* stream);
int mx_gemm_fp4_fp4_bias_gelu_quant(const void* a, const void* a_scale, const void* b,
                                    const void* b_scale, const void* bias, void* q, void* q_scale,
                                    int64_t M, int64_t N, int64_t K, void* stream);
int mx_gemm_fp4_fp4_bias_gelu_quant_strided_batched(const void* a, const void* a_scale,
                                                    const void* b, const void* b_scale,
                                                    const void* bias, void* q, void* q_scale,
                                                    int64_t M, int64_t N, int64_t K, int64_t batch,
                                                    int64_t stride_a, int64_t stride_a_scale,
                                                    int64_t stride_b, int64_t stride_b_scale,
                                                    int64_t stride_bias, int64_t stride_q,
                                                    int64_t stride_q_scale, void* stream);

/* ---------------------------------------------------------------------------------------------
 * GEMM with a residual or GELU epilogue (bf16 output).
 *
 * The "fp4-gemm README" page lists bias + residual and bias + GELU GEMM epilogues (API list; the
 * paragraph recommending fused epilogues so that consecutive low-bit GEMMs need no bf16 pass) without a
 * formula.  Here, with s[m,n] = sum_k A[m,k] B[n,k] (fp32 accumulation) and bias optional:
 *   _bias_residual:  c[m,n] = bf16_rne( s[m,n] + bias[n] + residual[m,n] )
 *   _bias_gelu:      c[m,n] = bf16_rne( gelu(s[m,n] + bias[n]) ),  gelu(x) = x * Phi(x) with Phi
 *                    the standard normal CDF (the exact form, not the tanh approximation)
 * one bf16 rounding each, all additions in fp32.
 *   bias      bf16 [N], or NULL (adds nothing)
 *   residual  bf16 [M, N] row-major (must not be NULL); it may be c itself (the same pointer and
 *             batch stride: an in-place residual add); any other overlap with c is undefined
 * Accuracy: the residual form meets the GEMM bound with ref = sum_k A B + bias + residual; the
 * GELU form satisfies |c - gelu(ref)| <= 2^-7 |gelu(ref)| + 2^-19 sum_k |A B| + 2^-126 with
 * ref = sum_k A B + bias (GELU's slope is at most 1.129).  Operands, formats, errors and the
 * other rules as for the plain entry points of the same kind.  Batched: residual +
 * i*stride_residual (bf16 elements; 0 reuses one residual for every batch).
 * ------------------------------------------------------------------------------------------- */
int mx_gemm_fp8_fp4_bias_residual(const void* a, const void* a_scale, const void* b,
                                  const void* b_scale, const void* bias, const void* residual,
                                  void* c, int64_t M, int64_t N, int64_t K, void* stream);
int mx_gemm_fp8_fp4_bias_residual_strided_batched(const void* a, const void* a_scale,
                                                  const void* b, const void* b_scale,
                                                  const void* bias, const void* residual, void* c,
                                                  int64_t M, int64_t N, int64_t K, int64_t batch,
                                                  int64_t stride_a, int64_t stride_a_scale,
                                                  int64_t stride_b, int64_t stride_b_scale,
                                                  int64_t stride_bias, int64_t stride_residual,
                                                  int64_t stride_c, void* stream);
int mx_gemm_fp8_fp4_bias_gelu(const void* a, const void* a_scale, const void* b,
                              const void* b_scale, const void* bias, void* c, int64_t M, int64_t N,
                              int64_t K, void* stream);
int mx_gemm_fp8_fp4_bias_gelu_strided_batched(const void* a, const void* a_scale, const void* b,
                                              const void* b_scale, const void* bias, void* c,
                                              int64_t M, int64_t N, int64_t K, int64_t batch,
                                              int64_t stride_a, int64_t stride_a_scale,
                                              int64_t stride_b, int64_t stride_b_scale,
                                              int64_t stride_bias, int64_t stride_c, void* stream);

int mx_gemm_fp8_fp8_bias_residual(const void* a, const void* a_scale, const void* b,
                                  const void* b_scale, const void* bias, const void* residual,
                                  void* c, int64_t M, int64_t N, int64_t K, void* stream);
int mx_gemm_fp8_fp8_bias_residual_strided_batched(const void* a, const void* a_scale,
                                                  const void* b, const void* b_scale,
                                                  const void* bias, const void* residual, void* c,
                                                  int64_t M, int64_t N, int64_t K, int64_t batch,
                                                  int64_t stride_a, int64_t stride_a_scale,
                                                  int64_t stride_b, int64_t stride_b_scale,
                                                  int64_t stride_bias, int64_t stride_residual,
                                                  int64_t stride_c, void* stream);
int mx_gemm_fp8_fp8_bias_gelu(const void* a, const void* a_scale, const void* b,
                              const void* b_scale, const void* bias, void* c, int64_t M, int64_t N,
                              int64_t K, void* stream);
int mx_gemm_fp8_fp8_bias_gelu_strided_batched(const void* a, const void* a_scale, const void* b,
                                              const void* b_scale, const void* bias, void* c,
                                              int64_t M, int64_t N, int64_t K, int64_t batch,
                                              int64_t stride_a, int64_t stride_a_scale,
                                              int64_t stride_b, int64_t stride_b_scale,
                                              int64_t stride_bias, int64_t stride_c, void* stream);

int mx_gemm_fp4_fp4_bias_residual(const void* a, const void* a_scale, const void* b,
                                  const void* b_scale, const void* bias, const void* residual,
                                  void* c, int64_t M, int64_t N, int64_t K, void* stream);
int mx_gemm_fp4_fp4_bias_residual_strided_batched(const void* a, const void* a_scale,
                                                  const void* b, const void* b_scale,
                                                  const void* bias, const void* residual, void* c,
                                                  int64_t M, int64_t N, int64_t K, int64_t batch,
                                                  int64_t stride_a, int64_t stride_a_scale,
                                                  int64_t stride_b, int64_t stride_b_scale,
                                                  int64_t stride_bias, int64_t stride_residual,
                                                  int64_t stride_c, void* stream);
int mx_gemm_fp4_fp4_bias_gelu(const void* a, const void* a_scale, const void* b,
                              const void* b_scale, const void* bias, void* c, int64_t M, int64_t N,
                              int64_t K, void* stream);
int mx_gemm_fp4_fp4_bias_gelu_strided_batched(const void* a, const void* a_scale, const void* b,
                                              const void* b_scale, const void* bias, void* c,
                                              int64_t M, int64_t N, int64_t K, int64_t batch,
                                              int64_t stride_a, int64_t stride_a_scale,
                                              int64_t stride_b, int64_t stride_b_scale,
                                              int64_t stride_bias, int64_t stride_c, void* stream);

/* ---------------------------------------------------------------------------------------------
 * Split-K GEMM for shapes with few output tiles and a long K (large down-projections).
 *
 * The "fp4-gemm README" page offers stream-K variants of its GEMM, which it uses only on the
 * large down-projection shapes (API list; the paragraph after the schedule variants).  Here the
 * load-balancing variant splits K: a single problem with 65..128 output tiles of 256 x 256
 * (fewer than the 256 CUs of an MI355X) and at least 80 K steps of 64 has each tile's K cut into
 * 2 equal ranges computed by separate workgroups.  The first of the two to finish stores its
 * fp32 partial tile in the workspace and raises the tile's ready flag; the other waits for the
 * flag (only ever for a workgroup that is already running and waits for nothing), adds that
 * partial to its own (fp32 addition commutes, so the bits do not depend on which came first),
 * adds the bias and rounds once to bf16.  A wait past about 2^22 polls, which no working device
 * reaches, gives up and writes NaN for that tile instead of hanging.  Shapes the plan does not
 * split (the skinny MXFP4 x MXFP4
 * shapes, M <= 64, among them) run exactly as mx_gemm_<kind>_bias (or without bias) do, and
 * need no workspace.
 *
 * mx_gemm_splitk_workspace_size: bytes of workspace an M x N x K call needs; 0 when that shape is
 *   not split (also for invalid sizes).  It depends on the shape alone (safe without a GPU).
 * mx_gemm_<kind>_splitk: as mx_gemm_<kind>_bias with bias optional (NULL: no bias), single
 *   problem, plus
 *   workspace        device memory of at least the size above, 256-byte aligned; before its
 *                    first use it must be zero-filled (its head holds a counter and a ready flag
 *                    per tile); every completed call leaves them zero again, so it can be reused
 *                    as is.  The rest holds one fp32 256 x 256 partial tile per output tile.
 *                    Calls sharing one workspace must not run concurrently.
 *   workspace_bytes  its size.  MX_ERR_WORKSPACE when a split shape gets a NULL, smaller or
 *                    misaligned workspace.
 * Accuracy: the bound of the plain GEMM (the partial sums are fp32, added in fp32).
 * ------------------------------------------------------------------------------------------- */
int64_t mx_gemm_splitk_workspace_size(int64_t M, int64_t N, int64_t K);
int mx_gemm_fp8_fp4_splitk(const void* a, const void* a_scale, const void* b, const void* b_scale,
                           const void* bias, void* c, int64_t M, int64_t N, int64_t K,
                           void* workspace, int64_t workspace_bytes, void* stream);
int mx_gemm_fp8_fp8_splitk(const void* a, const void* a_scale, const void* b, const void* b_scale,
                           const void* bias, void* c, int64_t M, int64_t N, int64_t K,
                           void* workspace, int64_t workspace_bytes, void* stream);
int mx_gemm_fp4_fp4_splitk(const void* a, const void* a_scale, const void* b, const void* b_scale,
                           const void* bias, void* c, int64_t M, int64_t N, int64_t K,
                           void* workspace, int64_t workspace_bytes, void* stream);

/* mx_gemm_fp8_fp4_splitk_noalloc: mx_gemm_fp8_fp4_splitk for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments without the workspace, the same kernels and results (bit for bit), and no
 * allocation of any kind.  The counters, ready flags and partial tiles live in a fixed device
 * array of this library, 32 MB + 1 KB, which every GPU the library runs on holds until the
 * process ends; it covers every shape the split plan splits (at most 128 output tiles), and a
 * plan that needed more would get MX_ERR_WORKSPACE.  Each call first clears the counters and
 * flags it uses with a small fill kernel on `stream`, then launches the GEMM; shapes that are
 * not split run as mx_gemm_fp8_fp4_bias (or without bias) and touch no array.  All calls on one
 * GPU share its array and it keeps the last call's contents, so calls that overlap on one GPU
 * (on concurrent streams, or from several threads) race: serialize them. */
int mx_gemm_fp8_fp4_splitk_noalloc(const void* a, const void* a_scale, const void* b,
                                   const void* b_scale, const void* bias, void* c, int64_t M,
                                   int64_t N, int64_t K, void* stream);

/* ---------------------------------------------------------------------------------------------
 * Backward-pass operands and GEMM (E5M2 gradients).
 *
 * The hip_quant page uses E4M3 for forward activations and weights and E5M2 (1 sign, 5 exponent
 * bits with bias 15, 2 mantissa bits, largest magnitude 57344; FP8 Formats table) for backward
 * gradients, rounded to nearest even or, opt-in, stochastically: between the two neighbouring
 * E5M2 values with chances that follow the distances, from a hash of the seed and the element's
 * index (section "Stochastic E5M2 Backward Gradients"); it also quantizes with a
 * fused transpose for rank-2 tensors.  The AstrAI page routes a linear layer's input and weight
 * gradients through the forward GEMM on transposed operands.  For y = x W^T (x [M, K], W [N, K]):
 *   dX [M, K] = dY W     = mx_gemm_e5m2_e4m3(quant_e5m2(dY) [M, N], quant_transpose_e4m3(W) [K, N])
 *   dW [N, K] = dY^T x   = mx_gemm_e5m2_e4m3(quant_transpose_e5m2(dY) [N, M],
 *                                           quant_transpose_e4m3(x) [K, M])
 *
 * mx_quant_e5m2: bf16 x [M, K] -> E5M2 codes q [M, K] + E8M0 bytes s [M, K/32], per 32 along K:
 *   E = ceil(log2(amax / 57344)) with amax floored at 2^-126 and E at -127 (byte E + 127); the
 *   codes round x / 2^E (exact) to nearest even (stochastic == 0) or stochastically (stochastic
 *   != 0): the larger neighbour when u < 2^32 (|y| - lo) / (hi - lo), u the 32-bit uniform of the
 *   element, word i & 7 (64-bit word (i & 7) / 2, low half first) of Philox4x64-10 block i >> 3
 *   under key (seed, 0), i the element's row-major index in the output (over all batches).
 *   Same buffer rules as mx_act_quant; batched: strides as mx_act_quant_strided_batched.
 * mx_quant_transpose_e4m3: bf16 x [R, C] -> E4M3 codes q [C, R] + E8M0 bytes s [C, R/32]: exactly
 *   mx_act_quant of x^T, without a transposed copy.
 * mx_quant_transpose_e5m2: bf16 x [R, C] -> mx_quant_e5m2 of x^T (codes [C, R], bytes [C, R/32]),
 *   the element index being the code's position in the [C, R] output.
 *   Both: R % 32 == 0 and C % 8 == 0 (MX_ERR_SHAPE), x and q 16-byte aligned (MX_ERR_ALIGN).
 * mx_gemm_e5m2_e4m3: C = bf16_rne(A B^T) with A E5M2 [M, K] + per-row-32 E8M0 [M, K/32] and B E4M3
 *   [N, K] + per-row-32 E8M0 [N, K/32] (the layout mx_quant_transpose_e4m3 writes), fp32
 *   accumulation, the same accuracy bound and buffer rules as mx_gemm_fp8_fp8; decoded values must
 *   be bf16 normals (E5M2 scale bytes >= 17).
 * ------------------------------------------------------------------------------------------- */
int mx_quant_e5m2(const void* x, void* q, void* s, int64_t M, int64_t K, int stochastic,
                  uint64_t seed, void* stream);
int mx_quant_e5m2_strided_batched(const void* x, void* q, void* s, int64_t M, int64_t K,
                                  int64_t batch, int64_t stride_x, int64_t stride_q,
                                  int64_t stride_s, int stochastic, uint64_t seed, void* stream);
int mx_quant_transpose_e4m3(const void* x, void* q, void* s, int64_t R, int64_t C, void* stream);
int mx_quant_transpose_e5m2(const void* x, void* q, void* s, int64_t R, int64_t C, int stochastic,
                            uint64_t seed, void* stream);
int mx_gemm_e5m2_e4m3(const void* a, const void* a_scale, const void* b, const void* b_scale,
                      void* c, int64_t M, int64_t N, int64_t K, void* stream);
/* As mx_gemm_e5m2_e4m3 with K split across workgroups for shapes with few output tiles (the
 * rules, workspace and errors of mx_gemm_fp8_fp4_splitk). */
int mx_gemm_e5m2_e4m3_splitk(const void* a, const void* a_scale, const void* b,
                             const void* b_scale, void* c, int64_t M, int64_t N, int64_t K,
                             void* workspace, int64_t workspace_bytes, void* stream);
int mx_gemm_e5m2_e4m3_strided_batched(const void* a, const void* a_scale, const void* b,
                                      const void* b_scale, void* c, int64_t M, int64_t N,
                                      int64_t K, int64_t batch, int64_t stride_a,
                                      int64_t stride_a_scale, int64_t stride_b,
                                      int64_t stride_b_scale, int64_t stride_c, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MX_H_ */
