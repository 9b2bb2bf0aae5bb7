/*
 * mpdt.h -- C ABI of libmpdt.so: tiled mixed-precision matrix
 * multiply-accumulate, the W8A8 linear layer and the quantisation steps
 * around them on AMD MI355X
 * (gfx950 / CDNA4).  Plain C: integers, device pointers, a stream handle.
 *
 * Operations and where they are defined:
 *   D = A x B + C on small matrices, low-precision inputs, FP32 accumulation:
 *     "Tensor Core" chapter of the CUDA advanced handbook, sections "What a
 *     Tensor Core does" and "Precision: FP16, BF16, TF32, FP8" (FP32
 *     accumulation because long low-precision sums lose accuracy quickly;
 *     INT8 inputs accumulate in INT32; FP8 needs per-tensor, per-row or
 *     per-block scale factors).  The handbook's wmma_gemm.cu program fixes
 *     the row-major A[M][K], B[K][N], C[M][N] convention used here.
 *   The batch-1 W8A8 linear layer: "NVIDIA A100: from chip to SIMT",
 *     sections 5.1 (symmetric INT8 quantisation, per-token activation scale
 *     s_x, per-output-channel weight scale s_w, zero point 0, INT32 sum,
 *     dequantisation once in the epilogue; weights stored [N][K] row-major,
 *     one output channel per row) and 5.2 (the launch wrapper takes the
 *     quantised activation, the weights, the activation scale by value, the
 *     weight-scale array, the output and a stream; dequantisation order is
 *     float(z) * s_x, then * s_w[o]).
 *
 * Conventions shared by every entry point:
 *   - Layout: all matrices row-major; ld* are leading dimensions in ELEMENTS
 *     (distance between the starts of consecutive rows), ld >= row length.
 *   - Memory: every pointer is a device pointer on the current HIP device.
 *     The caller owns all buffers; the library never allocates, frees,
 *     copies to the host or synchronises, and keeps no per-call state.
 *   - Asynchrony: work is enqueued on `stream` (a hipStream_t; NULL = the
 *     default stream) and the call returns.  Faults inside a kernel surface
 *     at the caller's next synchronisation.
 *   - Errors: every argument is validated on the host BEFORE anything is
 *     launched; on any non-success status nothing is written or launched.
 *     mpdt_last_error() returns a thread-local description of the last
 *     failure.
 *   - Sizes: M == 0 or N == 0 is a successful no-op.  K == 0 gives D = C
 *     (or 0 when C is NULL) for the GEMMs with a C operand, D = 0 for the
 *     FP8 GEMM and y = 0 (z = 0) for the GEMV.  Dimensions must be at most
 *     2^30 and each operand must span fewer than 2^46 bytes.
 *   - Alignment: only element alignment is required; faster 128-bit paths
 *     are chosen internally from the alignment of pointers and leading
 *     dimensions.
 *   - Aliasing: D must not overlap A, B (or scales / x / W).  C may be
 *     exactly D (same pointer, ldc == ldd) for an in-place update; any other
 *     overlap of C and D is rejected.
 *   - Threads: calls from several host threads are safe.
 *   - Device: the current device must be gfx950.
 */
#ifndef MPDT_H
#define MPDT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MPDT_SUCCESS = 0,
    MPDT_ERROR_INVALID_VALUE = 1,      /* NULL required pointer, negative or too large dim,
                                          ld smaller than the row, GEMV with M != 1 */
    MPDT_ERROR_MISALIGNED = 2,         /* pointer not aligned to its element size */
    MPDT_ERROR_ALIASING = 3,           /* output overlaps an input (other than D == C) */
    MPDT_ERROR_NO_DEVICE = 4,          /* no HIP device available */
    MPDT_ERROR_UNSUPPORTED_DEVICE = 5, /* current device is not gfx950 */
    MPDT_ERROR_LAUNCH = 6              /* the HIP runtime reported an error at launch */
} mpdt_status;

/* D[M x N] (FP32) = A[M x K] . B[K x N] + C[M x N] (FP32), FP32 accumulation.
 * A and B hold IEEE binary16 bit patterns.  The product sum starts from zero
 * and C is added once at the end, so when every partial sum is exactly
 * representable in FP32 (e.g. small integers) D is the correctly rounded
 * FP32 value of the exact result.  C may be NULL (treated as zero). */
mpdt_status gemm_f16(int64_t M, int64_t N, int64_t K,
                     const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                     const float* C, int64_t ldc, float* D, int64_t ldd, void* stream);

/* As gemm_f16 with bfloat16 bit patterns for A and B. */
mpdt_status gemm_bf16(int64_t M, int64_t N, int64_t K,
                      const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                      const float* C, int64_t ldc, float* D, int64_t ldd, void* stream);

/* 16-bit-output variants: the same D = A . B + C formed in FP32, then
 * rounded once (to nearest, ties to even) to the input format -- IEEE FP16
 * (subnormals kept, overflow to infinity) for gemm_f16_f16out, bfloat16 for
 * gemm_bf16_bf16out -- halving the bytes written ("Tensor Core" page, the
 * improvements listed after its WMMA exercise: write the result back as
 * BF16).  C stays FP32 (may be NULL); D holds 16-bit patterns. */
mpdt_status gemm_f16_f16out(int64_t M, int64_t N, int64_t K,
                            const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                            const float* C, int64_t ldc, uint16_t* D, int64_t ldd, void* stream);
mpdt_status gemm_bf16_bf16out(int64_t M, int64_t N, int64_t K,
                              const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                              const float* C, int64_t ldc, uint16_t* D, int64_t ldd, void* stream);

/* Activations of the fused GEMM epilogue. */
typedef enum {
    MPDT_ACT_NONE = 0,   /* identity */
    MPDT_ACT_RELU = 1,   /* v if v > 0, else +0 (NaN gives +0) */
    MPDT_ACT_GELU = 2,   /* v * Phi(v), Phi the standard normal CDF (erf form, not the
                            tanh approximation) */
    MPDT_ACT_SILU = 3    /* v / (1 + exp(-v)) */
} mpdt_act;

/* FP16 / BF16 GEMM with a fused bias + activation epilogue, the linear
 * layer's floating-point epilogue ("NVIDIA A100: from chip to SIMT",
 * section 5.1, adds the bias there) written together with D:
 *   v = acc + C[i][j]        (acc: A . B in FP32, as in gemm_f16 / gemm_bf16)
 *   v = v + bias[j]          (skipped when bias is NULL)
 *   D[i][j] = act(v)         (act: an mpdt_act; FP32 arithmetic)
 * then D is FP32 (d16 = 0) or rounded once, to nearest even, to the input
 * format (d16 = 1: FP16 for gemm_f16_bias_act, BF16 for gemm_bf16_bias_act).
 * Each step is an FP32 operation in this order (the additions are exact when
 * every value is a small integer; ReLU is exact).  GELU and SiLU are
 * evaluated in FP32 with the hardware base-2 exponential and reciprocal, GELU's
 * erfc by the Chebyshev fit of Numerical Recipes (section 6.2, fractional
 * error below 1.2e-7): the result is within 2^-20 (|v| + |act(v)|) of the
 * exact function of the computed v.  bias: N FP32 values (device pointer, 4-byte aligned, may be NULL; D
 * may not overlap it).  C may be NULL; C == D in place only with d16 = 0.
 * An act outside mpdt_act or d16 outside {0, 1} is MPDT_ERROR_INVALID_VALUE. */
mpdt_status gemm_f16_bias_act(int64_t M, int64_t N, int64_t K,
                              const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                              const float* C, int64_t ldc, const float* bias, int act,
                              void* D, int64_t ldd, int d16, void* stream);
mpdt_status gemm_bf16_bias_act(int64_t M, int64_t N, int64_t K,
                               const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                               const float* C, int64_t ldc, const float* bias, int act,
                               void* D, int64_t ldd, int d16, void* stream);

/* D[M x N] (INT32) = A[M x K] (INT8) . B[K x N] (INT8) + C (INT32), exact
 * as long as no partial sum leaves the INT32 range (K * 128^2 + |C| < 2^31
 * guarantees it).  C may be NULL. */
mpdt_status gemm_i8_i32(int64_t M, int64_t N, int64_t K,
                        const int8_t* A, int64_t lda, const int8_t* B, int64_t ldb,
                        const int32_t* C, int64_t ldc, int32_t* D, int64_t ldd, void* stream);

/* D[M x N] (BF16 bits, round to nearest even) =
 *     sum over 128-wide K blocks kb of (scale_a[i][kb] * scale_b[kb][j / 128]) *
 *         sum_{k in kb} A[i][k] . B[k][j]
 * A[M x K] and B[K x N] are OCP FP8 E4M3 ("FN": bias 7, max 448) bytes.
 * scale_a is M x ceil(K/128) FP32 (leading dimension ld_sa), one dequantisation
 * multiplier per row and 128-wide K block; scale_b is ceil(K/128) x
 * ceil(N/128) FP32 (leading dimension ld_sb), one per 128 x 128 block of B.
 * Partial blocks at the K and N edges use their own scale.  FP32
 * accumulation; there is no C operand. */
mpdt_status gemm_fp8_blockscaled(int64_t M, int64_t N, int64_t K,
                                 const uint8_t* A, int64_t lda,
                                 const float* scale_a, int64_t ld_sa,
                                 const uint8_t* B, int64_t ldb,
                                 const float* scale_b, int64_t ld_sb,
                                 uint16_t* D, int64_t ldd, void* stream);

/* FP8 formats ("Tensor Core" page, section "Precision": E4M3 for weights
 * and activations, E5M2 -- 5 exponent bits, 2 fraction bits, the range of
 * FP16 -- for gradients).  Both are the OCP encodings: E4M3 "FN" (bias 7, no
 * infinities, max 448), E5M2 (bias 15, infinities and NaNs at exponent 31,
 * max 57344). */
typedef enum { MPDT_FP8_E4M3 = 0, MPDT_FP8_E5M2 = 1 } mpdt_fp8_format;

/* gemm_fp8_blockscaled with each operand's format given (fmt_a, fmt_b: an
 * mpdt_fp8_format; any mix).  Same scales, accumulation and output.  Codes
 * that decode to infinity or NaN give undefined results. */
mpdt_status gemm_fp8_blockscaled_fmt(int64_t M, int64_t N, int64_t K,
                                     const uint8_t* A, int64_t lda, int fmt_a,
                                     const float* scale_a, int64_t ld_sa,
                                     const uint8_t* B, int64_t ldb, int fmt_b,
                                     const float* scale_b, int64_t ld_sb,
                                     uint16_t* D, int64_t ldd, void* stream);

/* FP8 GEMM with per-row / per-tensor scales (same section: FP8 scale factors
 * per tensor, per row or per block):
 *   D[i][j] = bf16_rne( (acc[i][j] * scale_a[i * inc_a]) * scale_b[j * inc_b] )
 * acc = sum_k A[i][k] * B[k][j] of the decoded FP8 values, in FP32 (the
 * exact products added in FP32 in an order of the kernel's choosing), then
 * two FP32 products in this order.  scale_a holds one value per row of A
 * (inc_a = 1) or one for the tensor (inc_a = 0); scale_b one per column of B
 * (inc_b = 1) or one (inc_b = 0).  Scales are read (must be non-NULL) even
 * when K = 0, which gives D = bf16(0 * ...).  Formats as above. */
mpdt_status gemm_fp8_rowscaled(int64_t M, int64_t N, int64_t K,
                               const uint8_t* A, int64_t lda, int fmt_a,
                               const float* scale_a, int64_t inc_a,
                               const uint8_t* B, int64_t ldb, int fmt_b,
                               const float* scale_b, int64_t inc_b,
                               uint16_t* D, int64_t ldd, void* stream);

/* Batch-1 W8A8 linear layer.  M must be 1.
 *   z[o] = sum_k x[k] * W[o][k]                      (INT32, exact)
 *   y[o] = bf16_rne( (float(z[o]) * x_scale) * w_scale[o] )   (two FP32 products,
 *                                                     in this order)
 * x: K INT8 values; W: N x K INT8 stored one output channel per row, leading
 * dimension ldw >= K; w_scale: N FP32; y: N BF16 bit patterns; z_out
 * (optional, may be NULL): N INT32 raw sums.  Exact while K * 128^2 < 2^31. */
mpdt_status gemv_w8a8(int64_t M, int64_t N, int64_t K,
                      const int8_t* x, float x_scale,
                      const int8_t* W, int64_t ldw, const float* w_scale,
                      uint16_t* y, int32_t* z_out, void* stream);

/* W8A8 linear layer for M >= 1 tokens (a small batch), each token with its
 * own activation scale, and an optional bias added after the dequantisation
 * ("NVIDIA A100: from chip to SIMT", section 5.1: the bias belongs in the
 * floating-point epilogue).  For every token m and output channel o:
 *   Z[m][o] = sum_k X[m][k] * W[o][k]                                (INT32, exact)
 *   Y[m][o] = bf16_rne( ((float(Z) * x_scale[m]) * w_scale[o]) + bias[o] )
 * each step one IEEE FP32 operation, in this order (the bias step is skipped
 * when bias is NULL).  X: M x K INT8 (ldx); W: N x K INT8, one output channel
 * per row (ldw); x_scale: M FP32; w_scale, bias: N FP32; Y: M x N BF16 bits
 * (ldy); Z (optional, may be NULL): M x N INT32 (ldz).  The weights are read
 * once per group of up to 32 tokens.  Exact while K * 128^2 < 2^31. */
mpdt_status gemm_w8a8(int64_t M, int64_t N, int64_t K,
                      const int8_t* X, int64_t ldx, const float* x_scale,
                      const int8_t* W, int64_t ldw, const float* w_scale, const float* bias,
                      uint16_t* Y, int64_t ldy, int32_t* Z, int64_t ldz, void* stream);

/* gemm_w8a8 with the weights stored K x N: W[k][o] at W + k * ldw + o,
 * ldw >= N (the logical [K][N] operand of x . W).  Same Z and Y, same
 * arithmetic; a K x N chunk of W is staged through LDS so that the matrix
 * instruction still gets K-consecutive bytes per channel. */
mpdt_status gemm_w8a8_kn(int64_t M, int64_t N, int64_t K,
                         const int8_t* X, int64_t ldx, const float* x_scale,
                         const int8_t* W, int64_t ldw, const float* w_scale, const float* bias,
                         uint16_t* Y, int64_t ldy, int32_t* Z, int64_t ldz, void* stream);

/* The same layer with a requantising epilogue, for a next layer that takes
 * INT8 (same section: the epilogue may requantise instead of writing a
 * 16-bit result).  With v the FP32 value whose BF16 rounding gemm_w8a8
 * writes (the same three or four FP32 steps, in the same order):
 *   Q[m][o] = clamp(rne(v / out_scale), -127, 127)     (INT8, ldq)
 * one IEEE FP32 division by the single output scale (symmetric, zero point
 * 0, as quantize_i8_rows; -128 is never produced), rne = round half to
 * even.  out_scale must be finite and > 0 (else MPDT_ERROR_INVALID_VALUE).
 * Z (optional) as in gemm_w8a8. */
mpdt_status gemm_w8a8_requant(int64_t M, int64_t N, int64_t K,
                              const int8_t* X, int64_t ldx, const float* x_scale,
                              const int8_t* W, int64_t ldw, const float* w_scale,
                              const float* bias, float out_scale,
                              int8_t* Q, int64_t ldq, int32_t* Z, int64_t ldz, void* stream);

/* Per-token symmetric INT8 quantisation of activations (the step that makes
 * the W8A8 layer's q_x and s_x; same section: symmetric, zero point 0, one
 * scale per token).  For each row m of the M x K BF16 matrix X (ldx):
 *   scales[m] = amax_k |X[m][k]| / 127   (FP32 division; 1 when the row is 0)
 *   Q[m][k]   = clamp(rne(X[m][k] / scales[m]), -127, 127)    (INT8, ldq)
 * rne = round to nearest, ties to even. */
mpdt_status quantize_i8_rows(int64_t M, int64_t K, const uint16_t* X, int64_t ldx,
                             int8_t* Q, int64_t ldq, float* scales, void* stream);

/* FP8 E4M3 block quantisation ("Tensor Core" page, section "Precision": FP8
 * needs scale factors per tensor, per row or per block).  The R x C FP32
 * matrix X (ldx) is cut into block_rows x 128 blocks (block_rows = 1 for the
 * 1 x 128 activation blocks, 128 for the 128 x 128 weight blocks of
 * gemm_fp8_blockscaled; edge blocks keep their own scale):
 *   s = amax_block |x| / 448   (FP32 division; 1 for an all-zero block)
 *   Q = e4m3_rne(x / s)        (OCP E4M3FN codes, ldq)
 * scales is ceil(R/block_rows) x ceil(C/128) FP32 with leading dimension lds
 * -- exactly the scale_a / scale_b operand of gemm_fp8_blockscaled. */
mpdt_status quantize_fp8_blocks(int64_t R, int64_t C, const float* X, int64_t ldx,
                                int64_t block_rows, uint8_t* Q, int64_t ldq,
                                float* scales, int64_t lds, void* stream);

/* FP8 quantisation with a choice of format and scale granularity (same
 * section: per tensor, per row or per block; E4M3 or E5M2):
 *   s = amax_block |x| / qmax   (qmax 448 for E4M3, 57344 for E5M2; FP32
 *                                division; 1 for an all-zero block)
 *   Q = fp8_rne(x / s)          (codes of fmt, ldq)
 * block_rows x block_cols may be 1 x 128 or 128 x 128 (as above), or cover
 * whole rows (1 x bc with bc >= C: one scale per row), whole columns
 * (br x 1 with br >= R: one per column) or the whole matrix (br >= R and
 * bc >= C: one per tensor); anything else is MPDT_ERROR_INVALID_VALUE.
 * scales is ceil(R/block_rows) x ceil(C/block_cols) (lds).  The per-tensor
 * form runs as several kernels on the stream and uses scales[0] as its
 * accumulator in between. */
mpdt_status quantize_fp8(int64_t R, int64_t C, const float* X, int64_t ldx, int fmt,
                         int64_t block_rows, int64_t block_cols, uint8_t* Q, int64_t ldq,
                         float* scales, int64_t lds, void* stream);

/* Static text for a status code. */
const char* mpdt_status_string(mpdt_status s);
/* Thread-local description of the last non-success status on this thread. */
const char* mpdt_last_error(void);
/* Library version: major * 10000 + minor * 100 + patch. */
int mpdt_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MPDT_H */
