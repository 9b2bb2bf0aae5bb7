/*
 * oracle.c -- plain, slow, obviously correct CPU oracle.  TEST INFRASTRUCTURE
 * ONLY (see oracle.h for what may call it and what each function follows).
 *
 * Build: gcc -std=c11 -O2 -fopenmp -ffp-contract=off -fPIC -shared
 * (-ffp-contract=off so that no multiply-add is fused behind our back; the
 * FP32 steps of the W8A8 dequantisation must be separate IEEE operations).
 *
 * Loops: every output element is an independent sum taken in ascending k, the
 * order of the definition.  The full-matrix functions walk i, then k, then j
 * (each R[i][j] still receives its terms in ascending k); OpenMP splits rows
 * between threads, which does not change any element's summation order.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Number formats, decoded exactly from their bit fields.                    */
/* ------------------------------------------------------------------------ */

/* FP16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
double oracle_f16_to_f64(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -24);            /* subnormal: f/2^10 * 2^-14 */
    } else if (e == 31) {
        v = (f == 0) ? INFINITY : NAN;
    } else {
        v = ldexp((double)(1024 + f), e - 25); /* (1 + f/2^10) * 2^(e-15) */
    }
    return sign ? -v : v;
}

/* BF16: 1 sign, 8 exponent (bias 127), 7 fraction bits. */
double oracle_bf16_to_f64(uint16_t b) {
    int sign = (b >> 15) & 1;
    int e = (b >> 7) & 0xff;
    int f = b & 0x7f;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -133);            /* f/2^7 * 2^-126 */
    } else if (e == 255) {
        v = (f == 0) ? INFINITY : NAN;
    } else {
        v = ldexp((double)(128 + f), e - 134); /* (1 + f/2^7) * 2^(e-127) */
    }
    return sign ? -v : v;
}

/* FP8 E4M3 (OCP "FN"): 1 sign, 4 exponent (bias 7), 3 fraction bits; no
 * infinities; exponent 15 with fraction 7 is NaN; largest finite 448. */
double oracle_e4m3_to_f64(uint8_t q) {
    int sign = (q >> 7) & 1;
    int e = (q >> 3) & 0xf;
    int f = q & 0x7;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -9);              /* f/2^3 * 2^-6 */
    } else if (e == 15 && f == 7) {
        v = NAN;
    } else {
        v = ldexp((double)(8 + f), e - 10);    /* (1 + f/2^3) * 2^(e-7) */
    }
    return sign ? -v : v;
}

/* FP32 -> BF16, round to nearest, ties to even.  BF16 keeps the upper 16 bits
 * of the FP32 encoding; the lower 16 bits are the discarded part.  Above half
 * an ulp rounds away from zero, below rounds toward zero, exactly half goes to
 * the even neighbour.  Carrying into the exponent is the correct next value
 * (and gives infinity past the largest finite).  NaN stays a quiet NaN. */
uint16_t oracle_f32_to_bf16_rne(float x) {
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    if (isnan(x)) return (uint16_t)(sign | 0x7fc0u);
    uint32_t mag = u & 0x7fffffffu;
    uint32_t kept = mag >> 16;
    uint32_t dropped = mag & 0xffffu;
    if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u))) kept += 1u;
    return (uint16_t)(sign | kept);
}

/* Exponent E of the binade of a > 0 (2^E <= a < 2^(E+1)). */
static int binade(double a) {
    int e;
    frexp(a, &e);   /* a = m * 2^e, m in [0.5, 1) */
    return e - 1;
}

/* FP32 -> FP16, round to nearest, ties to even.  A binade [2^E, 2^(E+1))
 * with E >= -14 holds 1024 values spaced 2^(E-10); below 2^-14 the spacing
 * is the subnormal quantum 2^-24.  The value is counted in quanta of its
 * binade (exact in double) and rounded with rint, which rounds to the
 * nearest integer, ties to even, in the default rounding mode.  A count of
 * 2048 is the first value of the next binade; past 65504 the result is
 * infinity. */
uint16_t oracle_f32_to_f16_rne(float x) {
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    if (isnan(x)) return (uint16_t)(sign | 0x7e00u);
    double a = fabs((double)x);
    if (a == 0.0) return sign;
    if (isinf(x)) return (uint16_t)(sign | 0x7c00u);
    int E = binade(a);
    if (E < -14) {
        double n = rint(ldexp(a, 24));          /* subnormal quanta, 0..1024 */
        return (uint16_t)(sign | (uint16_t)n);  /* 1024 encodes 2^-14 */
    }
    double n = rint(ldexp(a, 10 - E));          /* 1024..2048 */
    if (n == 2048.0) {
        n = 1024.0;
        E += 1;
    }
    if (E > 15) return (uint16_t)(sign | 0x7c00u);
    return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)(n - 1024.0));
}

/* FP32 -> E4M3FN, round to nearest, ties to even, saturating.  Normal
 * binades E = -6..8 hold 8 values spaced 2^(E-3); below 2^-6 the spacing is
 * 2^-9.  Anything that rounds beyond 448 (1.75 * 2^8, the largest finite
 * value) saturates to 448. */
uint8_t oracle_f32_to_e4m3_rne_sat(float x) {
    uint8_t sign = signbit(x) ? 0x80u : 0u;
    if (isnan(x)) return (uint8_t)(sign | 0x7fu);
    double a = fabs((double)x);
    if (a == 0.0) return sign;
    if (a >= 448.0) return (uint8_t)(sign | 0x7eu);
    int E = binade(a);
    if (E < -6) {
        double n = rint(ldexp(a, 9));           /* 0..8; 8 encodes 2^-6 */
        return (uint8_t)(sign | (uint8_t)n);
    }
    double n = rint(ldexp(a, 3 - E));           /* 8..16 */
    if (n == 16.0) {
        n = 8.0;
        E += 1;
    }
    if (E > 8 || (E == 8 && n > 14.0)) return (uint8_t)(sign | 0x7eu);
    return (uint8_t)(sign | (uint8_t)((E + 7) << 3) | (uint8_t)(n - 8.0));
}

/* FP8 E5M2 (OCP): 1 sign, 5 exponent (bias 15), 2 fraction bits; exponent
 * 31 holds the infinities (fraction 0) and NaNs; largest finite 57344. */
double oracle_e5m2_to_f64(uint8_t q) {
    int sign = (q >> 7) & 1;
    int e = (q >> 2) & 0x1f;
    int f = q & 0x3;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -16);             /* f/2^2 * 2^-14 */
    } else if (e == 31) {
        v = f ? NAN : INFINITY;
    } else {
        v = ldexp((double)(4 + f), e - 17);    /* (1 + f/2^2) * 2^(e-15) */
    }
    return sign ? -v : v;
}

/* FP32 -> E5M2, round to nearest, ties to even, saturating to +-57344
 * (1.75 * 2^15) instead of overflowing to infinity.  Normal binades
 * E = -14..15 hold 4 values spaced 2^(E-2); below 2^-14 the spacing is
 * 2^-16.  NaN gives S.11111.11. */
uint8_t oracle_f32_to_e5m2_rne_sat(float x) {
    uint8_t sign = signbit(x) ? 0x80u : 0u;
    if (isnan(x)) return (uint8_t)(sign | 0x7fu);
    double a = fabs((double)x);
    if (a == 0.0) return sign;
    if (a >= 57344.0) return (uint8_t)(sign | 0x7bu);
    int E = binade(a);
    if (E < -14) {
        double n = rint(ldexp(a, 16));          /* 0..4; 4 encodes 2^-14 */
        return (uint8_t)(sign | (uint8_t)n);
    }
    double n = rint(ldexp(a, 2 - E));           /* 4..8 */
    if (n == 8.0) {
        n = 4.0;
        E += 1;
    }
    if (E > 15) return (uint8_t)(sign | 0x7bu);
    return (uint8_t)(sign | (uint8_t)((E + 15) << 2) | (uint8_t)(n - 4.0));
}

void oracle_decode_e5m2(const uint8_t* in, double* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e5m2_to_f64(in[i]);
}

void oracle_decode_f16(const uint16_t* in, double* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f16_to_f64(in[i]);
}
void oracle_decode_bf16(const uint16_t* in, double* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_to_f64(in[i]);
}
void oracle_decode_e4m3(const uint8_t* in, double* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_to_f64(in[i]);
}
void oracle_round_bf16(const float* in, uint16_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f32_to_bf16_rne(in[i]);
}

/* ------------------------------------------------------------------------ */
/* Helpers: argument checks and dense decoding of a row-major operand.       */
/* ------------------------------------------------------------------------ */

static int dims_ok(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb) {
    if (M < 0 || N < 0 || K < 0) return 0;
    if (lda < (K > 0 ? K : 1) && M > 0 && K > 0) return 0;
    if (ldb < (N > 0 ? N : 1) && K > 0 && N > 0) return 0;
    return 1;
}

typedef double (*decode16_fn)(uint16_t);

/* Decode a rows x cols 16-bit operand (leading dimension ld) to a dense
 * double array; returns NULL on allocation failure or a non-finite value
 * (*bad set to 1 for the latter). */
static double* decode16_dense(const uint16_t* X, int64_t rows, int64_t cols, int64_t ld,
                              decode16_fn dec, int* bad) {
    size_t n = (size_t)(rows > 0 ? rows : 1) * (size_t)(cols > 0 ? cols : 1);
    double* out = (double*)malloc(n * sizeof(double));
    if (!out) return NULL;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            double v = dec(X[r * ld + c]);
            if (!isfinite(v)) *bad = 1;
            out[r * cols + c] = v;
        }
    return out;
}

/* ------------------------------------------------------------------------ */
/* FP16 / BF16 GEMM in FP64.                                                 */
/* ------------------------------------------------------------------------ */

static int gemm16(int64_t M, int64_t N, int64_t K,
                  const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                  const float* C, int64_t ldc, double* R, double* S, decode16_fn dec) {
    if (!dims_ok(M, N, K, lda, ldb) || !R || !S) return 1;
    if (C && M > 0 && N > 0 && ldc < N) return 1;
    if (M == 0 || N == 0) return 0;
    int bad = 0;
    double* Ad = decode16_dense(A, M, K, lda, dec, &bad);
    double* Bd = decode16_dense(B, K, N, ldb, dec, &bad);
    if (!Ad || !Bd) { free(Ad); free(Bd); return 1; }
    if (bad) { free(Ad); free(Bd); return 2; }
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i) {
        double* r = R + i * N;
        double* s = S + i * N;
        for (int64_t j = 0; j < N; ++j) { r[j] = 0.0; s[j] = 0.0; }
        for (int64_t k = 0; k < K; ++k) {
            const double a = Ad[i * K + k];
            const double* b = Bd + k * N;
            for (int64_t j = 0; j < N; ++j) {
                const double p = a * b[j];   /* exact: both factors have <= 11 significant bits */
                r[j] += p;
                s[j] += fabs(p);
            }
        }
        if (C)
            for (int64_t j = 0; j < N; ++j) r[j] += (double)C[i * ldc + j];
    }
    free(Ad);
    free(Bd);
    return 0;
}

int oracle_gemm_f16(int64_t M, int64_t N, int64_t K,
                    const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                    const float* C, int64_t ldc, double* R, double* S) {
    return gemm16(M, N, K, A, lda, B, ldb, C, ldc, R, S, oracle_f16_to_f64);
}
int oracle_gemm_bf16(int64_t M, int64_t N, int64_t K,
                     const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                     const float* C, int64_t ldc, double* R, double* S) {
    return gemm16(M, N, K, A, lda, B, ldb, C, ldc, R, S, oracle_bf16_to_f64);
}

/* One output element at a time: a dot product over k in ascending order. */
static int gemm16_at(int64_t M, int64_t N, int64_t K,
                     const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                     const float* C, int64_t ldc,
                     int64_t P, const int64_t* ii, const int64_t* jj, double* R, double* S,
                     decode16_fn dec) {
    if (!dims_ok(M, N, K, lda, ldb) || P < 0 || (P > 0 && (!ii || !jj || !R || !S))) return 1;
    int bad = 0;
    #pragma omp parallel for schedule(dynamic, 16) reduction(|:bad)
    for (int64_t p = 0; p < P; ++p) {
        const int64_t i = ii[p], j = jj[p];
        if (i < 0 || i >= M || j < 0 || j >= N) { bad |= 4; continue; }
        double r = 0.0, s = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double a = dec(A[i * lda + k]);
            const double b = dec(B[k * ldb + j]);
            if (!isfinite(a) || !isfinite(b)) bad |= 2;
            r += a * b;
            s += fabs(a * b);
        }
        if (C) r += (double)C[i * ldc + j];
        R[p] = r;
        S[p] = s;
    }
    if (bad & 4) return 1;
    if (bad & 2) return 2;
    return 0;
}

int oracle_gemm_f16_at(int64_t M, int64_t N, int64_t K,
                       const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                       const float* C, int64_t ldc,
                       int64_t P, const int64_t* ii, const int64_t* jj, double* R, double* S) {
    return gemm16_at(M, N, K, A, lda, B, ldb, C, ldc, P, ii, jj, R, S, oracle_f16_to_f64);
}
int oracle_gemm_bf16_at(int64_t M, int64_t N, int64_t K,
                        const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                        const float* C, int64_t ldc,
                        int64_t P, const int64_t* ii, const int64_t* jj, double* R, double* S) {
    return gemm16_at(M, N, K, A, lda, B, ldb, C, ldc, P, ii, jj, R, S, oracle_bf16_to_f64);
}

/* ------------------------------------------------------------------------ */
/* FP16 GEMM with integer-valued inputs: exact integer sum, one FP32 add.    */
/* ------------------------------------------------------------------------ */

int oracle_gemm_f16_intexact(int64_t M, int64_t N, int64_t K,
                             const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                             const float* C, int64_t ldc, float* D) {
    if (!dims_ok(M, N, K, lda, ldb) || !D) return 1;
    if (C && M > 0 && N > 0 && ldc < N) return 1;
    int err = 0;
    for (int64_t i = 0; i < M && !err; ++i)
        for (int64_t j = 0; j < N && !err; ++j) {
            int64_t sum = 0;
            for (int64_t k = 0; k < K; ++k) {
                const double a = oracle_f16_to_f64(A[i * lda + k]);
                const double b = oracle_f16_to_f64(B[k * ldb + j]);
                if (!isfinite(a) || !isfinite(b)) { err = 2; break; }
                if (a != floor(a) || b != floor(b) || fabs(a) > 2048.0 || fabs(b) > 2048.0) {
                    err = 4;
                    break;
                }
                sum += (int64_t)a * (int64_t)b;
            }
            if (err) break;
            if (sum > 16777216 || sum < -16777216) { err = 3; break; }
            const float fs = (float)sum;                 /* exact: |sum| <= 2^24 */
            const float c = C ? C[i * ldc + j] : 0.0f;
            volatile float d = fs + c;                    /* the single FP32 rounding */
            D[i * N + j] = d;
        }
    return err;
}

/* ------------------------------------------------------------------------ */
/* INT8 x INT8 -> INT32 GEMM.                                                */
/* ------------------------------------------------------------------------ */

static int i8_dot(int64_t K, const int8_t* A, int64_t lda, const int8_t* B, int64_t ldb,
                  const int32_t* C, int64_t ldc, int64_t i, int64_t j, int32_t* out) {
    int64_t sum = 0;
    for (int64_t k = 0; k < K; ++k) sum += (int64_t)A[i * lda + k] * (int64_t)B[k * ldb + j];
    if (C) sum += (int64_t)C[i * ldc + j];
    if (sum > INT32_MAX || sum < INT32_MIN) return 3;
    *out = (int32_t)sum;
    return 0;
}

int oracle_gemm_i8_i32(int64_t M, int64_t N, int64_t K,
                       const int8_t* A, int64_t lda, const int8_t* B, int64_t ldb,
                       const int32_t* C, int64_t ldc, int32_t* D) {
    if (!dims_ok(M, N, K, lda, ldb) || !D) return 1;
    if (C && M > 0 && N > 0 && ldc < N) return 1;
    int err = 0;
    #pragma omp parallel for schedule(static) reduction(|:err)
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j) err |= i8_dot(K, A, lda, B, ldb, C, ldc, i, j, &D[i * N + j]);
    return err ? 3 : 0;
}

int oracle_gemm_i8_i32_at(int64_t M, int64_t N, int64_t K,
                          const int8_t* A, int64_t lda, const int8_t* B, int64_t ldb,
                          const int32_t* C, int64_t ldc,
                          int64_t P, const int64_t* ii, const int64_t* jj, int32_t* D) {
    if (!dims_ok(M, N, K, lda, ldb) || P < 0 || (P > 0 && (!ii || !jj || !D))) return 1;
    int err = 0;
    #pragma omp parallel for schedule(dynamic, 16) reduction(|:err)
    for (int64_t p = 0; p < P; ++p) {
        if (ii[p] < 0 || ii[p] >= M || jj[p] < 0 || jj[p] >= N) { err |= 8; continue; }
        err |= i8_dot(K, A, lda, B, ldb, C, ldc, ii[p], jj[p], &D[p]);
    }
    if (err & 8) return 1;
    return err ? 3 : 0;
}

/* ------------------------------------------------------------------------ */
/* FP8 E4M3 block-scaled GEMM.                                               */
/* ------------------------------------------------------------------------ */

#define FP8_BLOCK 128

static int fp8_args_ok(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
                       const float* sA, int64_t ld_sa, const float* sB, int64_t ld_sb) {
    if (!dims_ok(M, N, K, lda, ldb)) return 0;
    const int64_t kb = (K + FP8_BLOCK - 1) / FP8_BLOCK;
    const int64_t nb = (N + FP8_BLOCK - 1) / FP8_BLOCK;
    if (K > 0 && M > 0 && (!sA || ld_sa < kb)) return 0;
    if (K > 0 && N > 0 && (!sB || ld_sb < nb)) return 0;
    return 1;
}

typedef double (*decode8_fn)(uint8_t);

/* 0: E4M3, 1: E5M2 */
static decode8_fn fp8_decoder(int fmt) {
    return fmt == 0 ? oracle_e4m3_to_f64 : fmt == 1 ? oracle_e5m2_to_f64 : NULL;
}

/* One element: for each K block, the block's raw FP8 product sum times the
 * product of the two block scales, summed over blocks in ascending order. */
static int fp8_element(int64_t K, const uint8_t* A, int64_t lda, decode8_fn da, const float* sA,
                       int64_t ld_sa, const uint8_t* B, int64_t ldb, decode8_fn db,
                       const float* sB, int64_t ld_sb, int64_t i, int64_t j, double* r_out,
                       double* s_out) {
    double r = 0.0, s = 0.0;
    int bad = 0;
    for (int64_t k0 = 0; k0 < K; k0 += FP8_BLOCK) {
        const int64_t kb = k0 / FP8_BLOCK;
        const double sa = (double)sA[i * ld_sa + kb];
        const double sb = (double)sB[kb * ld_sb + j / FP8_BLOCK];
        if (!isfinite(sa) || !isfinite(sb)) bad = 1;
        const int64_t k1 = (k0 + FP8_BLOCK < K) ? k0 + FP8_BLOCK : K;
        double blk = 0.0;
        for (int64_t k = k0; k < k1; ++k) {
            const double a = da(A[i * lda + k]);
            const double b = db(B[k * ldb + j]);
            if (!isfinite(a) || !isfinite(b)) bad = 1;
            blk += a * b;                                  /* exact products */
            s += fabs(a * sa) * fabs(b * sb);
        }
        r += (sa * sb) * blk;
    }
    *r_out = r;
    *s_out = s;
    return bad ? 2 : 0;
}

/* The whole matrix: for every (i, j) exactly the operations of fp8_element in
 * the same order (k ascending inside each 128-wide block, blocks ascending,
 * one scaled addition per block), walked row by row -- for row i and block
 * kb, the block sums of all j grow together, k by k -- so that B is read
 * along its rows from one decoded copy instead of down a column per element.
 * The results are bit-identical to fp8_element's (tests compare the two). */
int oracle_gemm_fp8_blockscaled_fmt(int64_t M, int64_t N, int64_t K,
                                    const uint8_t* A, int64_t lda, int fmt_a,
                                    const float* sA, int64_t ld_sa,
                                    const uint8_t* B, int64_t ldb, int fmt_b,
                                    const float* sB, int64_t ld_sb, double* R, double* S) {
    const decode8_fn da = fp8_decoder(fmt_a), db = fp8_decoder(fmt_b);
    if (!da || !db) return 1;
    if (!fp8_args_ok(M, N, K, lda, ldb, sA, ld_sa, sB, ld_sb) || !R || !S) return 1;
    if (M == 0 || N == 0) return 0;
    const int64_t nb = (N + FP8_BLOCK - 1) / FP8_BLOCK;
    double* Bd = (double*)malloc((size_t)(K > 0 ? K : 1) * (size_t)N * sizeof(double));
    if (!Bd) return 1;
    int bad = 0, nomem = 0;
    #pragma omp parallel for schedule(static) reduction(|:bad)
    for (int64_t k = 0; k < K; ++k)
        for (int64_t j = 0; j < N; ++j) {
            Bd[k * N + j] = db(B[k * ldb + j]);
            if (!isfinite(Bd[k * N + j])) bad = 1;
        }
    #pragma omp parallel reduction(|:bad, nomem)
    {
        double* ad = (double*)malloc((size_t)(K > 0 ? K : 1) * sizeof(double));
        double* blk = (double*)malloc((size_t)N * sizeof(double));
        if (!ad || !blk) nomem = 1;
        #pragma omp for schedule(static)
        for (int64_t i = 0; i < M; ++i) {
            double* r = R + i * N;
            double* s = S + i * N;
            for (int64_t j = 0; j < N; ++j) { r[j] = 0.0; s[j] = 0.0; }
            if (!ad || !blk) continue;
            for (int64_t k = 0; k < K; ++k) {
                ad[k] = da(A[i * lda + k]);
                if (!isfinite(ad[k])) bad = 1;
            }
            for (int64_t k0 = 0; k0 < K; k0 += FP8_BLOCK) {
                const int64_t kb = k0 / FP8_BLOCK;
                const int64_t k1 = (k0 + FP8_BLOCK < K) ? k0 + FP8_BLOCK : K;
                const double sa = (double)sA[i * ld_sa + kb];
                if (!isfinite(sa)) bad = 1;
                for (int64_t j = 0; j < N; ++j) blk[j] = 0.0;
                for (int64_t k = k0; k < k1; ++k) {
                    const double a = ad[k];
                    const double asa = fabs(a * sa);
                    const double* b = Bd + k * N;
                    for (int64_t jb = 0; jb < nb; ++jb) {
                        const double sb = (double)sB[kb * ld_sb + jb];
                        const int64_t j1 = (jb + 1) * FP8_BLOCK < N ? (jb + 1) * FP8_BLOCK : N;
                        for (int64_t j = jb * FP8_BLOCK; j < j1; ++j) {
                            blk[j] += a * b[j];                    /* exact products */
                            s[j] += asa * fabs(b[j] * sb);
                        }
                    }
                }
                for (int64_t jb = 0; jb < nb; ++jb) {
                    const double sb = (double)sB[kb * ld_sb + jb];
                    if (!isfinite(sb)) bad = 1;
                    const int64_t j1 = (jb + 1) * FP8_BLOCK < N ? (jb + 1) * FP8_BLOCK : N;
                    for (int64_t j = jb * FP8_BLOCK; j < j1; ++j) r[j] += (sa * sb) * blk[j];
                }
            }
        }
        free(ad);
        free(blk);
    }
    free(Bd);
    if (nomem) return 1;
    return bad ? 2 : 0;
}

int oracle_gemm_fp8_blockscaled_fmt_at(int64_t M, int64_t N, int64_t K,
                                       const uint8_t* A, int64_t lda, int fmt_a,
                                       const float* sA, int64_t ld_sa,
                                       const uint8_t* B, int64_t ldb, int fmt_b,
                                       const float* sB, int64_t ld_sb,
                                       int64_t P, const int64_t* ii, const int64_t* jj,
                                       double* R, double* S) {
    const decode8_fn da = fp8_decoder(fmt_a), db = fp8_decoder(fmt_b);
    if (!da || !db) return 1;
    if (!fp8_args_ok(M, N, K, lda, ldb, sA, ld_sa, sB, ld_sb) || P < 0) return 1;
    if (P > 0 && (!ii || !jj || !R || !S)) return 1;
    int err = 0;
    #pragma omp parallel for schedule(dynamic, 16) reduction(|:err)
    for (int64_t p = 0; p < P; ++p) {
        if (ii[p] < 0 || ii[p] >= M || jj[p] < 0 || jj[p] >= N) { err |= 8; continue; }
        err |= fp8_element(K, A, lda, da, sA, ld_sa, B, ldb, db, sB, ld_sb, ii[p], jj[p], &R[p],
                           &S[p]);
    }
    if (err & 8) return 1;
    return err ? 2 : 0;
}

int oracle_gemm_fp8_blockscaled(int64_t M, int64_t N, int64_t K,
                                const uint8_t* A, int64_t lda, const float* sA, int64_t ld_sa,
                                const uint8_t* B, int64_t ldb, const float* sB, int64_t ld_sb,
                                double* R, double* S) {
    return oracle_gemm_fp8_blockscaled_fmt(M, N, K, A, lda, 0, sA, ld_sa, B, ldb, 0, sB, ld_sb, R, S);
}

int oracle_gemm_fp8_blockscaled_at(int64_t M, int64_t N, int64_t K,
                                   const uint8_t* A, int64_t lda, const float* sA, int64_t ld_sa,
                                   const uint8_t* B, int64_t ldb, const float* sB, int64_t ld_sb,
                                   int64_t P, const int64_t* ii, const int64_t* jj,
                                   double* R, double* S) {
    return oracle_gemm_fp8_blockscaled_fmt_at(M, N, K, A, lda, 0, sA, ld_sa, B, ldb, 0, sB, ld_sb,
                                              P, ii, jj, R, S);
}

/* ------------------------------------------------------------------------ */
/* FP8 GEMM with per-row A and per-column B scales (see oracle.h).           */
/* ------------------------------------------------------------------------ */
static int fp8_row_element(int64_t K, const uint8_t* A, int64_t lda, decode8_fn da, double sa,
                           const uint8_t* B, int64_t ldb, decode8_fn db, double sb, int64_t i,
                           int64_t j, double* r_out, double* s_out) {
    double r = 0.0, s = 0.0;
    int bad = !isfinite(sa) || !isfinite(sb);
    for (int64_t k = 0; k < K; ++k) {
        const double a = da(A[i * lda + k]);
        const double b = db(B[k * ldb + j]);
        if (!isfinite(a) || !isfinite(b)) bad = 1;
        r += a * b;
        s += fabs(a * b);
    }
    *r_out = (sa * sb) * r;
    *s_out = fabs(sa * sb) * s;
    return bad ? 2 : 0;
}

int oracle_gemm_fp8_rowscaled_at(int64_t M, int64_t N, int64_t K,
                                 const uint8_t* A, int64_t lda, int fmt_a,
                                 const float* sA, int64_t inc_a,
                                 const uint8_t* B, int64_t ldb, int fmt_b,
                                 const float* sB, int64_t inc_b,
                                 int64_t P, const int64_t* ii, const int64_t* jj,
                                 double* R, double* S) {
    const decode8_fn da = fp8_decoder(fmt_a), db = fp8_decoder(fmt_b);
    if (!da || !db || !dims_ok(M, N, K, lda, ldb) || P < 0) return 1;
    if ((inc_a != 0 && inc_a != 1) || (inc_b != 0 && inc_b != 1)) return 1;
    if ((M > 0 && !sA) || (N > 0 && !sB)) return 1;
    if (P > 0 && (!ii || !jj || !R || !S)) return 1;
    int err = 0;
    #pragma omp parallel for schedule(dynamic, 16) reduction(|:err)
    for (int64_t p = 0; p < P; ++p) {
        if (ii[p] < 0 || ii[p] >= M || jj[p] < 0 || jj[p] >= N) { err |= 8; continue; }
        err |= fp8_row_element(K, A, lda, da, (double)sA[ii[p] * inc_a], B, ldb, db,
                               (double)sB[jj[p] * inc_b], ii[p], jj[p], &R[p], &S[p]);
    }
    if (err & 8) return 1;
    return err ? 2 : 0;
}

int oracle_gemm_fp8_rowscaled(int64_t M, int64_t N, int64_t K,
                              const uint8_t* A, int64_t lda, int fmt_a,
                              const float* sA, int64_t inc_a,
                              const uint8_t* B, int64_t ldb, int fmt_b,
                              const float* sB, int64_t inc_b, double* R, double* S) {
    const decode8_fn da = fp8_decoder(fmt_a), db = fp8_decoder(fmt_b);
    if (!da || !db || !dims_ok(M, N, K, lda, ldb) || !R || !S) return 1;
    if ((inc_a != 0 && inc_a != 1) || (inc_b != 0 && inc_b != 1)) return 1;
    if ((M > 0 && !sA) || (N > 0 && !sB)) return 1;
    int err = 0;
    #pragma omp parallel for schedule(dynamic, 4) reduction(|:err)
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j)
            err |= fp8_row_element(K, A, lda, da, (double)sA[i * inc_a], B, ldb, db,
                                   (double)sB[j * inc_b], i, j, &R[i * N + j], &S[i * N + j]);
    return err ? 2 : 0;
}

/* ------------------------------------------------------------------------ */
/* Batch-1 W8A8 linear layer.                                                */
/* ------------------------------------------------------------------------ */

int oracle_gemv_w8a8(int64_t N, int64_t K, const int8_t* x, float s_x,
                     const int8_t* W, int64_t ldw, const float* s_w,
                     int32_t* z, uint16_t* y) {
    if (N < 0 || K < 0 || (N > 0 && (!y || !s_w)) || (N > 0 && K > 0 && (!x || !W || ldw < K)))
        return 1;
    int err = 0;
    #pragma omp parallel for schedule(static) reduction(|:err)
    for (int64_t o = 0; o < N; ++o) {
        int64_t acc = 0;
        for (int64_t k = 0; k < K; ++k) acc += (int64_t)x[k] * (int64_t)W[o * ldw + k];
        if (acc > INT32_MAX || acc < INT32_MIN) { err |= 1; continue; }
        if (z) z[o] = (int32_t)acc;
        /* Three separate IEEE single-precision steps, left to right. */
        volatile float t = (float)(int32_t)acc;
        t = t * s_x;
        t = t * s_w[o];
        y[o] = oracle_f32_to_bf16_rne(t);
    }
    return err ? 3 : 0;
}

/* ------------------------------------------------------------------------ */
/* M-token W8A8 layer with optional bias (see oracle.h).                      */
/* ------------------------------------------------------------------------ */
int oracle_gemm_w8a8(int64_t M, int64_t N, int64_t K, const int8_t* X, int64_t ldx,
                     const float* s_x, const int8_t* W, int64_t ldw, const float* s_w,
                     const float* bias, int32_t* Z, int64_t ldz, uint16_t* Y, int64_t ldy) {
    if (M < 0 || N < 0 || K < 0 || !X || !s_x || !W || !s_w || !Y) return 1;
    if ((M > 0 && K > 0 && ldx < K) || (N > 0 && K > 0 && ldw < K) || ldy < N ||
        (Z && ldz < N))
        return 1;
    for (int64_t m = 0; m < M; ++m)
        if (!isfinite(s_x[m])) return 2;
    for (int64_t o = 0; o < N; ++o)
        if (!isfinite(s_w[o]) || (bias && !isfinite(bias[o]))) return 2;
    int rc = 0;
#pragma omp parallel for schedule(static) reduction(max : rc)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t o = 0; o < N; ++o) {
            int64_t acc = 0;
            for (int64_t k = 0; k < K; ++k)
                acc += (int64_t)X[m * ldx + k] * (int64_t)W[o * ldw + k];
            if (acc > INT32_MAX || acc < INT32_MIN) {
                rc = 3;
                continue;
            }
            /* float(z) rounds to nearest (exact for |z| <= 2^24), then two
             * FP32 products and the bias, each an IEEE operation rounded once */
            float t = (float)(int32_t)acc;
            t = t * s_x[m];
            t = t * s_w[o];
            if (bias) t = t + bias[o];
            if (Z) Z[m * ldz + o] = (int32_t)acc;
            Y[m * ldy + o] = oracle_f32_to_bf16_rne(t);
        }
    }
    return rc;
}

/* ------------------------------------------------------------------------ */
/* M-token W8A8 layer, requantised to INT8 (see oracle.h).                    */
/* ------------------------------------------------------------------------ */
int oracle_gemm_w8a8_requant(int64_t M, int64_t N, int64_t K, const int8_t* X, int64_t ldx,
                             const float* s_x, const int8_t* W, int64_t ldw, const float* s_w,
                             const float* bias, float s_out, int32_t* Z, int64_t ldz,
                             int8_t* Q, int64_t ldq) {
    if (M < 0 || N < 0 || K < 0 || !X || !s_x || !W || !s_w || !Q) return 1;
    if ((M > 0 && K > 0 && ldx < K) || (N > 0 && K > 0 && ldw < K) || ldq < N ||
        (Z && ldz < N))
        return 1;
    if (!isfinite(s_out) || !(s_out > 0.0f)) return 1;
    for (int64_t m = 0; m < M; ++m)
        if (!isfinite(s_x[m])) return 2;
    for (int64_t o = 0; o < N; ++o)
        if (!isfinite(s_w[o]) || (bias && !isfinite(bias[o]))) return 2;
    int rc = 0;
#pragma omp parallel for schedule(static) reduction(max : rc)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t o = 0; o < N; ++o) {
            int64_t acc = 0;
            for (int64_t k = 0; k < K; ++k)
                acc += (int64_t)X[m * ldx + k] * (int64_t)W[o * ldw + k];
            if (acc > INT32_MAX || acc < INT32_MIN) {
                rc = 3;
                continue;
            }
            float t = (float)(int32_t)acc;
            t = t * s_x[m];
            t = t * s_w[o];
            if (bias) t = t + bias[o];
            /* one FP32 division, then round half to even (rint in the default
             * rounding mode) and saturate to the symmetric INT8 range */
            const float u = t / s_out;
            double r = rint((double)u);
            if (r > 127.0) r = 127.0;
            if (r < -127.0) r = -127.0;
            if (Z) Z[m * ldz + o] = (int32_t)acc;
            Q[m * ldq + o] = (int8_t)r;
        }
    }
    return rc;
}

/* ------------------------------------------------------------------------ */
/* Per-token INT8 quantisation (see oracle.h).                                */
/* ------------------------------------------------------------------------ */
int oracle_quantize_i8_rows(int64_t M, int64_t K, const uint16_t* X, int64_t ldx,
                            int8_t* Q, int64_t ldq, float* S) {
    if (M < 0 || K < 0 || !X || !Q || !S || (K > 0 && (ldx < K || ldq < K))) return 1;
    for (int64_t m = 0; m < M; ++m) {
        double amax = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double v = oracle_bf16_to_f64(X[m * ldx + k]);
            if (!isfinite(v)) return 2;
            if (fabs(v) > amax) amax = fabs(v);
        }
        /* amax is a BF16 value, exact in FP32 */
        float s = (amax > 0.0) ? (float)amax / 127.0f : 1.0f;
        S[m] = s;
        for (int64_t k = 0; k < K; ++k) {
            float t = (float)oracle_bf16_to_f64(X[m * ldx + k]) / s;
            double r = rint((double)t);
            if (r > 127.0) r = 127.0;
            if (r < -127.0) r = -127.0;
            Q[m * ldq + k] = (int8_t)r;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* FP8 E4M3 block quantisation (see oracle.h).                                */
/* ------------------------------------------------------------------------ */
int oracle_quantize_fp8_blocks_fmt(int64_t R, int64_t Cc, const float* X, int64_t ldx, int fmt,
                                   int64_t br, int64_t bc, uint8_t* Q, int64_t ldq,
                                   float* S, int64_t lds) {
    if (R < 0 || Cc < 0 || br < 1 || bc < 1 || !X || !Q || !S || (fmt != 0 && fmt != 1)) return 1;
    /* the largest finite value of the format */
    const float qmax = fmt == 0 ? 448.0f : 57344.0f;
    const int64_t nbr = (R + br - 1) / br, nbc = (Cc + bc - 1) / bc;
    if (Cc > 0 && (ldx < Cc || ldq < Cc)) return 1;
    if (nbc > 0 && lds < nbc) return 1;
    for (int64_t i = 0; i < R; ++i)
        for (int64_t j = 0; j < Cc; ++j)
            if (!isfinite(X[i * ldx + j])) return 2;
    for (int64_t bi = 0; bi < nbr; ++bi) {
        for (int64_t bj = 0; bj < nbc; ++bj) {
            const int64_t i0 = bi * br, i1 = (i0 + br < R) ? i0 + br : R;
            const int64_t j0 = bj * bc, j1 = (j0 + bc < Cc) ? j0 + bc : Cc;
            float amax = 0.0f;
            for (int64_t i = i0; i < i1; ++i)
                for (int64_t j = j0; j < j1; ++j)
                    if (fabsf(X[i * ldx + j]) > amax) amax = fabsf(X[i * ldx + j]);
            const float s = (amax > 0.0f) ? amax / qmax : 1.0f;
            S[bi * lds + bj] = s;
            for (int64_t i = i0; i < i1; ++i)
                for (int64_t j = j0; j < j1; ++j) {
                    const float u = X[i * ldx + j] / s;
                    Q[i * ldq + j] = fmt == 0 ? oracle_f32_to_e4m3_rne_sat(u) : oracle_f32_to_e5m2_rne_sat(u);
                }
        }
    }
    return 0;
}

int oracle_quantize_fp8_blocks(int64_t R, int64_t Cc, const float* X, int64_t ldx,
                               int64_t br, int64_t bc, uint8_t* Q, int64_t ldq,
                               float* S, int64_t lds) {
    return oracle_quantize_fp8_blocks_fmt(R, Cc, X, ldx, 0, br, bc, Q, ldq, S, lds);
}

/* ------------------------------------------------------------------------ */
/* Bias and activation epilogue (see oracle.h).                               */
/* ------------------------------------------------------------------------ */
static double act_of(double v, int act) {
    switch (act) {
        case 1: return v > 0.0 ? v : 0.0;
        /* Phi(v) = erfc(-v / sqrt 2) / 2: the same function as (1 + erf) / 2
         * without its cancellation for negative v */
        case 2: return 0.5 * v * erfc(-v / sqrt(2.0));
        case 3: return v / (1.0 + exp(-v));
        default: return v;
    }
}

int oracle_bias_act(int64_t M, int64_t N, double* R, int64_t ldr, const float* bias, int act) {
    if (M < 0 || N < 0 || !R || act < 0 || act > 3 || (M > 0 && ldr < N)) return 1;
    if (bias)
        for (int64_t j = 0; j < N; ++j)
            if (!isfinite(bias[j])) return 2;
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j) {
            double v = R[i * ldr + j];
            if (bias) v += (double)bias[j];
            R[i * ldr + j] = act_of(v, act);
        }
    return 0;
}
