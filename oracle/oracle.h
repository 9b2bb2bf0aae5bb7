/*
 * oracle.h -- plain CPU oracle for the tiled mixed-precision multiply-accumulate
 * D = A x B + C and the batch-1 W8A8 linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link or
 * call this library.  Its only users are the test-suite, the smoke check of the
 * package entry point and the CPU-baseline leg of the benchmark.  It shares no
 * source with the HIP kernels: it has its own number-format decoders, its own
 * BF16 rounding and its own loops.
 *
 * What it computes (each function below names the passage it follows):
 *   - GEMMs are the textbook sum D[i][j] = sum_k A[i][k] * B[k][j] + C[i][j]
 *     ("Tensor Core" handbook page, section "What a Tensor Core does": one
 *     instruction computes D = A x B + C on small matrices; the wmma_gemm.cu
 *     program indexes A and B row-major with leading dimension = row length).
 *     Floating point is accumulated in FP64 (exact products for FP16/BF16/E4M3
 *     inputs), integers in INT64.  Every floating-point GEMM also returns the
 *     bound matrix S[i][j] = sum_k |A[i][k] * B[k][j]| used by the tolerance.
 *   - Number formats FP16 (1/5/10), BF16 (1/8/7) and FP8 E4M3 (1/4/3) follow
 *     the format table of the same page, section "Precision: FP16, BF16, TF32,
 *     FP8".  E4M3 is the OCP "FN" variant (bias 7, no infinities, only
 *     S.1111.111 is NaN, largest finite 448).
 *   - The W8A8 linear layer follows "NVIDIA A100: from chip to SIMT", sections
 *     5.1 and 5.2: symmetric INT8 x INT8 products summed exactly in INT32, then
 *     one dequantisation in the epilogue, (float(z) * s_x) * s_w[o], in that
 *     left-to-right order; the weights are stored [N][K] row-major (one output
 *     channel per row).  Output is rounded to BF16 (round to nearest even).
 *
 * All matrices are row-major with explicit leading dimensions (in elements).
 * Output arrays R and S are dense M x N row-major (leading dimension N).
 *
 * Return codes: 0 ok, 1 invalid argument, 2 non-finite input, 3 integer
 * overflow of the INT32 result, 4 non-integer input to an exact-integer path.
 */
#ifndef MPDT_ORACLE_H
#define MPDT_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- number formats: exact decode to double, and FP32 -> BF16 RNE ---- */
double   oracle_f16_to_f64(uint16_t h);
double   oracle_bf16_to_f64(uint16_t b);
double   oracle_e4m3_to_f64(uint8_t q);
uint16_t oracle_f32_to_bf16_rne(float x);
/* FP32 -> IEEE FP16, round to nearest, ties to even, with subnormals;
 * overflow gives infinity.  (Format table of the "Tensor Core" page,
 * section "Precision": FP16 1/5/10.) */
uint16_t oracle_f32_to_f16_rne(float x);
/* FP32 -> OCP E4M3FN, round to nearest, ties to even, saturating to +-448
 * (no infinities in the format; NaN gives S.1111.111). */
uint8_t  oracle_f32_to_e4m3_rne_sat(float x);
/* OCP E5M2 (the "Precision" section's other FP8 format: 1/5/2 bits, wider
 * range, for gradients): exact decode (infinities and NaNs at exponent 31),
 * and FP32 -> E5M2 round to nearest, ties to even, saturating to +-57344. */
double   oracle_e5m2_to_f64(uint8_t q);
uint8_t  oracle_f32_to_e5m2_rne_sat(float x);
void     oracle_decode_e5m2(const uint8_t* in, double* out, int64_t n);

void oracle_decode_f16(const uint16_t* in, double* out, int64_t n);
void oracle_decode_bf16(const uint16_t* in, double* out, int64_t n);
void oracle_decode_e4m3(const uint8_t* in, double* out, int64_t n);
void oracle_round_bf16(const float* in, uint16_t* out, int64_t n);

/* ---- FP16 / BF16 GEMM, FP64 accumulation.  C may be NULL (= 0). ---- */
int oracle_gemm_f16(int64_t M, int64_t N, int64_t K,
                    const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                    const float* C, int64_t ldc, double* R, double* S);
int oracle_gemm_bf16(int64_t M, int64_t N, int64_t K,
                     const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                     const float* C, int64_t ldc, double* R, double* S);

/* Same sum at P listed output positions (rows ii[p], columns jj[p]). */
int oracle_gemm_f16_at(int64_t M, int64_t N, int64_t K,
                       const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                       const float* C, int64_t ldc,
                       int64_t P, const int64_t* ii, const int64_t* jj, double* R, double* S);
int oracle_gemm_bf16_at(int64_t M, int64_t N, int64_t K,
                        const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                        const float* C, int64_t ldc,
                        int64_t P, const int64_t* ii, const int64_t* jj, double* R, double* S);

/* FP16 GEMM whose inputs are all integers: the product sum is formed exactly
 * in INT64 (must fit 2^24 in magnitude) and C is added with ONE IEEE FP32
 * addition.  D is M x N FP32 (leading dimension N). */
int oracle_gemm_f16_intexact(int64_t M, int64_t N, int64_t K,
                             const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                             const float* C, int64_t ldc, float* D);

/* ---- INT8 x INT8 -> INT32 GEMM, exact (INT64 sum, checked to fit INT32). ---- */
int oracle_gemm_i8_i32(int64_t M, int64_t N, int64_t K,
                       const int8_t* A, int64_t lda, const int8_t* B, int64_t ldb,
                       const int32_t* C, int64_t ldc, int32_t* D);
int oracle_gemm_i8_i32_at(int64_t M, int64_t N, int64_t K,
                          const int8_t* A, int64_t lda, const int8_t* B, int64_t ldb,
                          const int32_t* C, int64_t ldc,
                          int64_t P, const int64_t* ii, const int64_t* jj, int32_t* D);

/* ---- FP8 E4M3 block-scaled GEMM (block 128 along K; B scales per 128x128).
 * R[i][j] = sum_kb (sA[i][kb] * sB[kb][j/128]) * sum_{k in block kb} a[i][k]*b[k][j]
 * S[i][j] = sum_k |a[i][k]*sA[i][k/128]| * |b[k][j]*sB[k/128][j/128]|
 * sA is M x ceil(K/128) (leading dimension ld_sa), sB is ceil(K/128) x
 * ceil(N/128) (leading dimension ld_sb). ---- */
/* The same with each operand's FP8 format given (fmt 0: E4M3, 1: E5M2). */
int oracle_gemm_fp8_blockscaled_fmt(int64_t M, int64_t N, int64_t K,
                                    const uint8_t* A, int64_t lda, int fmt_a,
                                    const float* sA, int64_t ld_sa,
                                    const uint8_t* B, int64_t ldb, int fmt_b,
                                    const float* sB, int64_t ld_sb, double* R, double* S);
int oracle_gemm_fp8_blockscaled_fmt_at(int64_t M, int64_t N, int64_t K,
                                       const uint8_t* A, int64_t lda, int fmt_a,
                                       const float* sA, int64_t ld_sa,
                                       const uint8_t* B, int64_t ldb, int fmt_b,
                                       const float* sB, int64_t ld_sb,
                                       int64_t P, const int64_t* ii, const int64_t* jj,
                                       double* R, double* S);

/* ---- FP8 GEMM with per-row / per-tensor scales (the "Precision" section:
 * FP8 scale factors per tensor, per row or per block): one scale per row of
 * A (sA[i * inc_a]) and one per column of B (sB[j * inc_b]); inc 0 makes
 * the scale per tensor.
 * R[i][j] = (sA[i*inc_a] * sB[j*inc_b]) * sum_k a[i][k] * b[k][j]
 * S[i][j] = |sA * sB| * sum_k |a[i][k] * b[k][j]|.  inc_a, inc_b in {0, 1}. ---- */
int oracle_gemm_fp8_rowscaled(int64_t M, int64_t N, int64_t K,
                              const uint8_t* A, int64_t lda, int fmt_a,
                              const float* sA, int64_t inc_a,
                              const uint8_t* B, int64_t ldb, int fmt_b,
                              const float* sB, int64_t inc_b, double* R, double* S);
int oracle_gemm_fp8_rowscaled_at(int64_t M, int64_t N, int64_t K,
                                 const uint8_t* A, int64_t lda, int fmt_a,
                                 const float* sA, int64_t inc_a,
                                 const uint8_t* B, int64_t ldb, int fmt_b,
                                 const float* sB, int64_t inc_b,
                                 int64_t P, const int64_t* ii, const int64_t* jj,
                                 double* R, double* S);

int oracle_gemm_fp8_blockscaled(int64_t M, int64_t N, int64_t K,
                                const uint8_t* A, int64_t lda, const float* sA, int64_t ld_sa,
                                const uint8_t* B, int64_t ldb, const float* sB, int64_t ld_sb,
                                double* R, double* S);
int oracle_gemm_fp8_blockscaled_at(int64_t M, int64_t N, int64_t K,
                                   const uint8_t* A, int64_t lda, const float* sA, int64_t ld_sa,
                                   const uint8_t* B, int64_t ldb, const float* sB, int64_t ld_sb,
                                   int64_t P, const int64_t* ii, const int64_t* jj,
                                   double* R, double* S);

/* ---- batch-1 W8A8 linear layer.
 * z[o] = sum_k x[k] * W[o][k] (exact), y[o] = bf16_rne((float(z[o]) * s_x) * s_w[o]).
 * W is N x K row-major with leading dimension ldw; z and y have N entries.
 * z may be NULL. ---- */
int oracle_gemv_w8a8(int64_t N, int64_t K, const int8_t* x, float s_x,
                     const int8_t* W, int64_t ldw, const float* s_w,
                     int32_t* z, uint16_t* y);

/* ---- M-token W8A8 linear layer (the same layer for M >= 1 tokens, each
 * with its own per-token activation scale), with an optional bias added in
 * the dequantised floating-point epilogue ("NVIDIA A100: from chip to SIMT",
 * section 5.1: a bias is added after dequantisation).
 * Z[m][o] = sum_k X[m][k] * W[o][k] (exact);
 * Y[m][o] = bf16_rne( fl32( fl32( fl32(float(Z) * s_x[m]) * s_w[o] ) + bias[o] ) )
 * (the bias step is skipped when bias is NULL).  X is M x K (ldx), W is N x K
 * (ldw); Z (may be NULL) and Y are M x N with leading dimensions ldz, ldy. ---- */
int oracle_gemm_w8a8(int64_t M, int64_t N, int64_t K, const int8_t* X, int64_t ldx,
                     const float* s_x, const int8_t* W, int64_t ldw, const float* s_w,
                     const float* bias, int32_t* Z, int64_t ldz, uint16_t* Y, int64_t ldy);

/* ---- The same M-token W8A8 layer with a requantising epilogue: the output
 * is INT8 for a next layer that takes INT8 (same section: instead of
 * writing FP16 the epilogue may requantise).  t is the FP32 value whose
 * BF16 rounding oracle_gemm_w8a8 writes, t = fl32(fl32(fl32(float(Z) *
 * s_x[m]) * s_w[o]) + bias[o]) (bias step skipped when bias is NULL); then
 * Q[m][o] = clamp(rne(fl32(t / s_out)), -127, 127) with one output scale
 * s_out (finite, > 0), symmetric with zero point 0 like the activation
 * quantiser below.  Z may be NULL.  Returns 1 for bad arguments (s_out not
 * finite and positive included). ---- */
int oracle_gemm_w8a8_requant(int64_t M, int64_t N, int64_t K, const int8_t* X, int64_t ldx,
                             const float* s_x, const int8_t* W, int64_t ldw, const float* s_w,
                             const float* bias, float s_out, int32_t* Z, int64_t ldz,
                             int8_t* Q, int64_t ldq);

/* ---- Per-token symmetric INT8 quantisation of activations (the step that
 * produces q_x and s_x upstream of the W8A8 layer, same section: symmetric,
 * zero point 0, one scale per token).  For each row m of the M x K BF16
 * matrix X: amax = max_k |X[m][k]|; s = fl32(amax / 127) (s = 1 when
 * amax = 0); Q[m][k] = clamp(rne(fl32(X[m][k] / s)), -127, 127).  S[m] = s. ---- */
int oracle_quantize_i8_rows(int64_t M, int64_t K, const uint16_t* X, int64_t ldx,
                            int8_t* Q, int64_t ldq, float* S);

/* ---- FP8 E4M3 block quantisation (the scale factors FP8 needs, "per tensor,
 * per row or per block", "Tensor Core" page, section "Precision").  The
 * R x Cc FP32 matrix X is cut into br x bc blocks (partial blocks at the
 * edges keep their own scale); for each block amax = max |x|,
 * s = fl32(amax / 448) (s = 1 when amax = 0), Q = e4m3_rne_sat(fl32(x / s)).
 * S is ceil(R/br) x ceil(Cc/bc) with leading dimension lds. ---- */
/* The same into E4M3 (fmt 0, s = amax / 448) or E5M2 (fmt 1, s = amax /
 * 57344); br x bc blocks of any size: 1 x Cc is one scale per row, R x Cc one
 * per tensor. */
int oracle_quantize_fp8_blocks_fmt(int64_t R, int64_t Cc, const float* X, int64_t ldx, int fmt,
                                   int64_t br, int64_t bc, uint8_t* Q, int64_t ldq,
                                   float* S, int64_t lds);
int oracle_quantize_fp8_blocks(int64_t R, int64_t Cc, const float* X, int64_t ldx,
                               int64_t br, int64_t bc, uint8_t* Q, int64_t ldq,
                               float* S, int64_t lds);

/* ---- Bias and activation after a FP16 / BF16 GEMM (the fused epilogue of
 * the 16-bit GEMM entry points).  In place on an M x N FP64 result R
 * (leading dimension ldr): R[i][j] = act(R[i][j] + bias[j]), the bias being
 * one FP32 value per output column ("NVIDIA A100: from chip to SIMT",
 * section 5.1: a linear layer's bias is added in the floating-point
 * epilogue; bias may be NULL: no add).  act: 0 identity, 1 ReLU
 * (v if v > 0, else 0), 2 GELU (v * Phi(v), Phi the standard normal CDF,
 * Phi(v) = erfc(-v / sqrt 2) / 2 = (1 + erf(v / sqrt 2)) / 2), 3 SiLU (v / (1 + exp(-v))).
 * Returns 1 for an unknown act or bad arguments, 2 for a non-finite bias. ---- */
int oracle_bias_act(int64_t M, int64_t N, double* R, int64_t ldr, const float* bias, int act);

#ifdef __cplusplus
}
#endif
#endif /* MPDT_ORACLE_H */
