// abi.hip -- the C ABI of libmpdt.so (declared in include/mpdt.h): host-side
// argument validation, device check, kernel selection and launch.  No device
// code lives here.  Every check runs before anything is launched.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <mutex>
#include <string>

#include "kernels.hpp"
#include "mpdt.h"

static_assert(MPDT_ACT_NONE == mpdt::ACT_NONE && MPDT_ACT_RELU == mpdt::ACT_RELU &&
                  MPDT_ACT_GELU == mpdt::ACT_GELU && MPDT_ACT_SILU == mpdt::ACT_SILU,
              "activation codes of the C ABI and the kernels agree");

#define MPDT_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

constexpr int64_t kMaxDim = int64_t(1) << 30;
constexpr int64_t kMaxSpanBytes = int64_t(1) << 46;

thread_local std::string g_last_error;

mpdt_status fail(mpdt_status s, const char* fn, const char* what) {
    char buf[256];
    snprintf(buf, sizeof buf, "%s: %s", fn, what);
    g_last_error = buf;
    return s;
}

struct Span {
    uintptr_t lo = 0, hi = 0;   // [lo, hi) bytes; empty when lo == hi
    bool overlaps(const Span& o) const { return lo < o.hi && o.lo < hi && lo != hi && o.lo != o.hi; }
};

// Byte span of a rows x cols operand with leading dimension ld (elements).
// Returns false when it does not fit the size limit.
bool span_of(const void* p, int64_t rows, int64_t cols, int64_t ld, int64_t es, Span* out) {
    *out = Span{};
    if (rows <= 0 || cols <= 0) return true;
    const int64_t lim = kMaxSpanBytes / es;
    if (ld > lim) return false;
    if (rows > 1 && (ld > 0) && (rows - 1) > (lim - cols) / ld) return false;
    const int64_t elems = (rows - 1) * ld + cols;
    out->lo = reinterpret_cast<uintptr_t>(p);
    out->hi = out->lo + (uintptr_t)(elems * es);
    return true;
}

bool aligned_to(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Current device must be a gfx950; the answer is cached per device.
constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
int g_is_gfx950[kMaxDevices];

mpdt_status check_device(const char* fn) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return fail(MPDT_ERROR_NO_DEVICE, fn, "no HIP device available");
    }
    if (dev >= kMaxDevices) return fail(MPDT_ERROR_UNSUPPORTED_DEVICE, fn, "device index too large");
    std::call_once(g_once[dev], [dev] {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
            (void)hipGetLastError();
            g_is_gfx950[dev] = 0;
            return;
        }
        g_is_gfx950[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    });
    if (!g_is_gfx950[dev]) return fail(MPDT_ERROR_UNSUPPORTED_DEVICE, fn, "current device is not gfx950");
    return MPDT_SUCCESS;
}

mpdt_status launched(hipError_t e, const char* fn) {
    if (e == hipSuccess) return MPDT_SUCCESS;
    return fail(MPDT_ERROR_LAUNCH, fn, hipGetErrorString(e));
}

bool dims_ok(int64_t M, int64_t N, int64_t K) {
    return M >= 0 && N >= 0 && K >= 0 && M <= kMaxDim && N <= kMaxDim && K <= kMaxDim;
}

// Shared validation of the three GEMMs with A[MxK], B[KxN], optional C and D.
mpdt_status check_gemm(const char* fn, int64_t M, int64_t N, int64_t K, const void* A,
                       int64_t lda, int64_t esa, const void* B, int64_t ldb, int64_t esb,
                       const void* C, int64_t ldc, int64_t esc, const void* D, int64_t ldd,
                       int64_t esd, Span extra_inputs[], int n_extra) {
    if (!dims_ok(M, N, K)) return fail(MPDT_ERROR_INVALID_VALUE, fn, "dimension out of range");
    if (M == 0 || N == 0) return MPDT_SUCCESS;
    if (!D) return fail(MPDT_ERROR_INVALID_VALUE, fn, "D is NULL");
    if (ldd < N) return fail(MPDT_ERROR_INVALID_VALUE, fn, "ldd < N");
    if (K > 0) {
        if (!A || !B) return fail(MPDT_ERROR_INVALID_VALUE, fn, "A or B is NULL");
        if (lda < K) return fail(MPDT_ERROR_INVALID_VALUE, fn, "lda < K");
        if (ldb < N) return fail(MPDT_ERROR_INVALID_VALUE, fn, "ldb < N");
    }
    if (C && ldc < N) return fail(MPDT_ERROR_INVALID_VALUE, fn, "ldc < N");
    if (!aligned_to(D, esd) || (C && !aligned_to(C, esc)) ||
        (K > 0 && (!aligned_to(A, esa) || !aligned_to(B, esb))))
        return fail(MPDT_ERROR_MISALIGNED, fn, "pointer not aligned to its element size");
    Span sa, sb, sc, sd;
    if (!span_of(D, M, N, ldd, esd, &sd) || !span_of(C, C ? M : 0, N, ldc, esc, &sc) ||
        (K > 0 && (!span_of(A, M, K, lda, esa, &sa) || !span_of(B, K, N, ldb, esb, &sb))))
        return fail(MPDT_ERROR_INVALID_VALUE, fn, "operand too large");
    if (sd.overlaps(sa) || sd.overlaps(sb))
        return fail(MPDT_ERROR_ALIASING, fn, "D overlaps A or B");
    for (int i = 0; i < n_extra; ++i)
        if (sd.overlaps(extra_inputs[i])) return fail(MPDT_ERROR_ALIASING, fn, "D overlaps a scale or bias array");
    if (C && sd.overlaps(sc) && !(C == D && ldc == ldd))
        return fail(MPDT_ERROR_ALIASING, fn, "C overlaps D without being exactly D");
    return MPDT_SUCCESS;
}

// FP16 / BF16 GEMM; D is FP32 (out16 = 0) or in the input format (out16 = 1).
mpdt_status run_gemm16(const char* fn, mpdt::Kind kind, int64_t M, int64_t N, int64_t K,
                       const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                       const float* C, int64_t ldc, void* D, int64_t ldd, int out16,
                       void* stream, bool fused = false, const float* bias = nullptr, int act = 0) {
    if (out16 != 0 && out16 != 1) return fail(MPDT_ERROR_INVALID_VALUE, fn, "d16 must be 0 or 1");
    if (fused && (act < MPDT_ACT_NONE || act > MPDT_ACT_SILU))
        return fail(MPDT_ERROR_INVALID_VALUE, fn, "unknown activation");
    const int64_t esd = out16 ? 2 : 4;
    // a 16-bit D cannot be updated in place from an FP32 C
    if (out16 && C && (const void*)C == (const void*)D)
        return fail(MPDT_ERROR_ALIASING, fn, "C may not alias a 16-bit D");
    Span sbias;   // the bias: N FP32 values, an input D may not overlap
    if (!span_of(bias, bias && M > 0 ? 1 : 0, N, N, 4, &sbias))
        return fail(MPDT_ERROR_INVALID_VALUE, fn, "operand too large");
    mpdt_status s = check_gemm(fn, M, N, K, A, lda, 2, B, ldb, 2, C, ldc, 4, D, ldd, esd, &sbias,
                               bias ? 1 : 0);
    if (s != MPDT_SUCCESS || M == 0 || N == 0) return s;
    if (bias && !aligned_to(bias, 4))
        return fail(MPDT_ERROR_MISALIGNED, fn, "bias not aligned to 4 bytes");
    if ((s = check_device(fn)) != MPDT_SUCCESS) return s;
    mpdt::GemmArgs a{};
    a.A = (const char*)A;
    a.B = (const char*)B;
    a.C = C;
    a.D = D;
    a.lda_b = lda * 2;
    a.ldb_b = ldb * 2;
    a.ldc = ldc;
    a.ldd = ldd;
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    a.out16 = out16;
    a.d16_vec = out16 && aligned_to(D, 16) && (ldd * 2) % 16 == 0;
    a.bias = bias;
    a.act = act;
    const bool al = aligned_to(A, 16) && aligned_to(B, 16) && (a.lda_b % 16 == 0) &&
                    (a.ldb_b % 16 == 0);
    if (fused) return launched(mpdt::launch_gemm_epi(kind, a, al, (hipStream_t)stream), fn);
    return launched(mpdt::launch_gemm(kind, a, al, (hipStream_t)stream), fn);
}

}  // namespace

MPDT_EXPORT mpdt_status gemm_f16(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda,
                                 const uint16_t* B, int64_t ldb, const float* C, int64_t ldc,
                                 float* D, int64_t ldd, void* stream) {
    return run_gemm16("gemm_f16", mpdt::Kind::F16, M, N, K, A, lda, B, ldb, C, ldc, D, ldd, 0,
                      stream);
}

MPDT_EXPORT mpdt_status gemm_f16_f16out(int64_t M, int64_t N, int64_t K, const uint16_t* A,
                                        int64_t lda, const uint16_t* B, int64_t ldb, const float* C,
                                        int64_t ldc, uint16_t* D, int64_t ldd, void* stream) {
    return run_gemm16("gemm_f16_f16out", mpdt::Kind::F16, M, N, K, A, lda, B, ldb, C, ldc, D, ldd,
                      1, stream);
}

MPDT_EXPORT mpdt_status gemm_bf16_bf16out(int64_t M, int64_t N, int64_t K, const uint16_t* A,
                                          int64_t lda, const uint16_t* B, int64_t ldb,
                                          const float* C, int64_t ldc, uint16_t* D, int64_t ldd,
                                          void* stream) {
    return run_gemm16("gemm_bf16_bf16out", mpdt::Kind::BF16, M, N, K, A, lda, B, ldb, C, ldc, D,
                      ldd, 1, stream);
}

MPDT_EXPORT mpdt_status gemm_bf16(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda,
                                  const uint16_t* B, int64_t ldb, const float* C, int64_t ldc,
                                  float* D, int64_t ldd, void* stream) {
    return run_gemm16("gemm_bf16", mpdt::Kind::BF16, M, N, K, A, lda, B, ldb, C, ldc, D, ldd, 0,
                      stream);
}

MPDT_EXPORT mpdt_status gemm_f16_bias_act(int64_t M, int64_t N, int64_t K, const uint16_t* A,
                                          int64_t lda, const uint16_t* B, int64_t ldb,
                                          const float* C, int64_t ldc, const float* bias, int act,
                                          void* D, int64_t ldd, int d16, void* stream) {
    return run_gemm16("gemm_f16_bias_act", mpdt::Kind::F16, M, N, K, A, lda, B, ldb, C, ldc, D, ldd,
                      d16, stream, true, bias, act);
}

MPDT_EXPORT mpdt_status gemm_bf16_bias_act(int64_t M, int64_t N, int64_t K, const uint16_t* A,
                                           int64_t lda, const uint16_t* B, int64_t ldb,
                                           const float* C, int64_t ldc, const float* bias, int act,
                                           void* D, int64_t ldd, int d16, void* stream) {
    return run_gemm16("gemm_bf16_bias_act", mpdt::Kind::BF16, M, N, K, A, lda, B, ldb, C, ldc, D,
                      ldd, d16, stream, true, bias, act);
}

MPDT_EXPORT mpdt_status gemm_i8_i32(int64_t M, int64_t N, int64_t K, const int8_t* A, int64_t lda,
                                    const int8_t* B, int64_t ldb, const int32_t* C, int64_t ldc,
                                    int32_t* D, int64_t ldd, void* stream) {
    const char* fn = "gemm_i8_i32";
    mpdt_status s = check_gemm(fn, M, N, K, A, lda, 1, B, ldb, 1, C, ldc, 4, D, ldd, 4, nullptr, 0);
    if (s != MPDT_SUCCESS || M == 0 || N == 0) return s;
    if ((s = check_device(fn)) != MPDT_SUCCESS) return s;
    mpdt::GemmArgs a{};
    a.A = (const char*)A;
    a.B = (const char*)B;
    a.C = C;
    a.D = D;
    a.lda_b = lda;
    a.ldb_b = ldb;
    a.ldc = ldc;
    a.ldd = ldd;
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    const bool al = aligned_to(A, 16) && aligned_to(B, 16) && lda % 16 == 0 && ldb % 16 == 0;
    return launched(mpdt::launch_gemm(mpdt::Kind::I8, a, al, (hipStream_t)stream), fn);
}

namespace {
// The FP8 GEMMs.  Block-scaled: scale_a M x ceil(K/128) (ld_sa), scale_b
// ceil(K/128) x ceil(N/128) (ld_sb).  Row-scaled (rows): scale_a holds M
// values read with increment ld_sa (0 or 1), scale_b N values with
// increment ld_sb.
mpdt_status run_fp8(const char* fn, int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda,
                    int fmt_a, const float* scale_a, int64_t ld_sa, const uint8_t* B, int64_t ldb,
                    int fmt_b, const float* scale_b, int64_t ld_sb, bool rows, uint16_t* D,
                    int64_t ldd, void* stream) {
    if (!dims_ok(M, N, K)) return fail(MPDT_ERROR_INVALID_VALUE, fn, "dimension out of range");
    if ((fmt_a != MPDT_FP8_E4M3 && fmt_a != MPDT_FP8_E5M2) ||
        (fmt_b != MPDT_FP8_E4M3 && fmt_b != MPDT_FP8_E5M2))
        return fail(MPDT_ERROR_INVALID_VALUE, fn, "unknown FP8 format");
    if (rows && ((ld_sa != 0 && ld_sa != 1) || (ld_sb != 0 && ld_sb != 1)))
        return fail(MPDT_ERROR_INVALID_VALUE, fn, "scale increments must be 0 or 1");
    const int64_t kb = (K + 127) / 128, nb = (N + 127) / 128;
    Span ssa, ssb;
    if (M > 0 && N > 0 && (K > 0 || rows)) {
        if (!scale_a || !scale_b) return fail(MPDT_ERROR_INVALID_VALUE, fn, "scale array is NULL");
        if (!aligned_to(scale_a, 4) || !aligned_to(scale_b, 4))
            return fail(MPDT_ERROR_MISALIGNED, fn, "scale array not 4-byte aligned");
        if (rows) {
            if (!span_of(scale_a, 1, ld_sa ? M : 1, M, 4, &ssa) ||
                !span_of(scale_b, 1, ld_sb ? N : 1, N, 4, &ssb))
                return fail(MPDT_ERROR_INVALID_VALUE, fn, "scale array too large");
        } else {
            if (ld_sa < kb) return fail(MPDT_ERROR_INVALID_VALUE, fn, "ld_sa < ceil(K/128)");
            if (ld_sb < nb) return fail(MPDT_ERROR_INVALID_VALUE, fn, "ld_sb < ceil(N/128)");
            if (!span_of(scale_a, M, kb, ld_sa, 4, &ssa) || !span_of(scale_b, kb, nb, ld_sb, 4, &ssb))
                return fail(MPDT_ERROR_INVALID_VALUE, fn, "scale array too large");
        }
    }
    Span extra[2] = {ssa, ssb};
    mpdt_status s = check_gemm(fn, M, N, K, A, lda, 1, B, ldb, 1, nullptr, 0, 4, D, ldd, 2, extra, 2);
    if (s != MPDT_SUCCESS || M == 0 || N == 0) return s;
    if ((s = check_device(fn)) != MPDT_SUCCESS) return s;
    mpdt::GemmArgs a{};
    a.A = (const char*)A;
    a.B = (const char*)B;
    a.C = nullptr;
    a.D = D;
    a.lda_b = lda;
    a.ldb_b = ldb;
    a.ldc = 0;
    a.ldd = ldd;
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    a.sA = scale_a;
    a.ld_sa = ld_sa;
    a.sB = scale_b;
    a.ld_sb = ld_sb;
    a.fp8_fmt = (fmt_a == MPDT_FP8_E5M2 ? 1 : 0) | (fmt_b == MPDT_FP8_E5M2 ? 2 : 0);
    a.row_scaled = rows ? 1 : 0;
    const bool al = aligned_to(A, 16) && aligned_to(B, 16) && lda % 16 == 0 && ldb % 16 == 0;
    return launched(mpdt::launch_fp8(a, al, (hipStream_t)stream), fn);
}
}  // namespace

MPDT_EXPORT mpdt_status gemm_fp8_blockscaled(int64_t M, int64_t N, int64_t K, const uint8_t* A,
                                             int64_t lda, const float* scale_a, int64_t ld_sa,
                                             const uint8_t* B, int64_t ldb, const float* scale_b,
                                             int64_t ld_sb, uint16_t* D, int64_t ldd,
                                             void* stream) {
    return run_fp8("gemm_fp8_blockscaled", M, N, K, A, lda, MPDT_FP8_E4M3, scale_a, ld_sa, B, ldb,
                   MPDT_FP8_E4M3, scale_b, ld_sb, false, D, ldd, stream);
}

MPDT_EXPORT mpdt_status gemm_fp8_blockscaled_fmt(int64_t M, int64_t N, int64_t K, const uint8_t* A,
                                                 int64_t lda, int fmt_a, const float* scale_a,
                                                 int64_t ld_sa, const uint8_t* B, int64_t ldb,
                                                 int fmt_b, const float* scale_b, int64_t ld_sb,
                                                 uint16_t* D, int64_t ldd, void* stream) {
    return run_fp8("gemm_fp8_blockscaled_fmt", M, N, K, A, lda, fmt_a, scale_a, ld_sa, B, ldb, fmt_b,
                   scale_b, ld_sb, false, D, ldd, stream);
}

MPDT_EXPORT mpdt_status gemm_fp8_rowscaled(int64_t M, int64_t N, int64_t K, const uint8_t* A,
                                           int64_t lda, int fmt_a, const float* scale_a,
                                           int64_t inc_a, const uint8_t* B, int64_t ldb, int fmt_b,
                                           const float* scale_b, int64_t inc_b, uint16_t* D,
                                           int64_t ldd, void* stream) {
    return run_fp8("gemm_fp8_rowscaled", M, N, K, A, lda, fmt_a, scale_a, inc_a, B, ldb, fmt_b,
                   scale_b, inc_b, true, D, ldd, stream);
}

MPDT_EXPORT mpdt_status gemv_w8a8(int64_t M, int64_t N, int64_t K, const int8_t* x, float x_scale,
                                  const int8_t* W, int64_t ldw, const float* w_scale, uint16_t* y,
                                  int32_t* z_out, void* stream) {
    const char* fn = "gemv_w8a8";
    if (!dims_ok(M, N, K)) return fail(MPDT_ERROR_INVALID_VALUE, fn, "dimension out of range");
    if (M != 1) return fail(MPDT_ERROR_INVALID_VALUE, fn, "M must be 1 (batch-1 layer)");
    if (N == 0) return MPDT_SUCCESS;
    if (!y || !w_scale) return fail(MPDT_ERROR_INVALID_VALUE, fn, "y or w_scale is NULL");
    if (K > 0) {
        if (!x || !W) return fail(MPDT_ERROR_INVALID_VALUE, fn, "x or W is NULL");
        if (ldw < K) return fail(MPDT_ERROR_INVALID_VALUE, fn, "ldw < K");
    }
    if (!aligned_to(y, 2) || !aligned_to(w_scale, 4) || (z_out && !aligned_to(z_out, 4)))
        return fail(MPDT_ERROR_MISALIGNED, fn, "pointer not aligned to its element size");
    Span sx, sw, ss, sy, sz;
    if (!span_of(W, K > 0 ? N : 0, K, ldw, 1, &sw) || !span_of(x, K > 0 ? 1 : 0, K, K, 1, &sx) ||
        !span_of(w_scale, 1, N, N, 4, &ss) || !span_of(y, 1, N, N, 2, &sy) ||
        !span_of(z_out, z_out ? 1 : 0, N, N, 4, &sz))
        return fail(MPDT_ERROR_INVALID_VALUE, fn, "operand too large");
    if (sy.overlaps(sx) || sy.overlaps(sw) || sy.overlaps(ss) || sz.overlaps(sx) ||
        sz.overlaps(sw) || sz.overlaps(ss) || sz.overlaps(sy))
        return fail(MPDT_ERROR_ALIASING, fn, "an output overlaps an input or the other output");
    mpdt_status s = check_device(fn);
    if (s != MPDT_SUCCESS) return s;
    mpdt::GemvArgs a{};
    a.x = x;
    a.W = W;
    a.ldw = ldw;
    a.w_scale = w_scale;
    a.y = y;
    a.z = z_out;
    a.x_scale = x_scale;
    a.N = (int)N;
    a.K = (int)K;
    const bool al = aligned_to(x, 16) && aligned_to(W, 16) && ldw % 16 == 0;
    return launched(mpdt::launch_gemv_w8a8(a, al, (hipStream_t)stream), fn);
}

namespace {
// The M-token W8A8 layer; the output is BF16 Y, or INT8 Q requantised by
// out_scale (requant).
mpdt_status run_w8a8(const char* fn, int64_t M, int64_t N, int64_t K, const int8_t* X, int64_t ldx,
                     const float* x_scale, const int8_t* W, int64_t ldw, const float* w_scale,
                     const float* bias, void* Y, int64_t ldy, bool requant, float out_scale,
                     int32_t* Z, int64_t ldz, void* stream, bool w_kn = false) {
    const int64_t esy = requant ? 1 : 2;
    if (!dims_ok(M, N, K)) return fail(MPDT_ERROR_INVALID_VALUE, fn, "dimension out of range");
    if (requant && !(std::isfinite(out_scale) && out_scale > 0.0f))
        return fail(MPDT_ERROR_INVALID_VALUE, fn, "out_scale must be finite and positive");
    if (M == 0 || N == 0) return MPDT_SUCCESS;
    if (!Y || !x_scale || !w_scale)
        return fail(MPDT_ERROR_INVALID_VALUE, fn, "output, x_scale or w_scale is NULL");
    if (K > 0) {
        if (!X || !W) return fail(MPDT_ERROR_INVALID_VALUE, fn, "X or W is NULL");
        if (ldx < K) return fail(MPDT_ERROR_INVALID_VALUE, fn, "ldx < K");
        if (ldw < (w_kn ? N : K)) return fail(MPDT_ERROR_INVALID_VALUE, fn, w_kn ? "ldw < N" : "ldw < K");
    }
    if (ldy < N || (Z && ldz < N)) return fail(MPDT_ERROR_INVALID_VALUE, fn, "output ld or ldz < N");
    if (!aligned_to(Y, esy) || !aligned_to(x_scale, 4) || !aligned_to(w_scale, 4) ||
        (bias && !aligned_to(bias, 4)) || (Z && !aligned_to(Z, 4)))
        return fail(MPDT_ERROR_MISALIGNED, fn, "pointer not aligned to its element size");
    Span sx, sw, ssx, ssw, sb, sy, sz;
    if (!span_of(X, K > 0 ? M : 0, K, ldx, 1, &sx) ||
        !(w_kn ? span_of(W, K, N, ldw, 1, &sw) : span_of(W, K > 0 ? N : 0, K, ldw, 1, &sw)) ||
        !span_of(x_scale, 1, M, M, 4, &ssx) || !span_of(w_scale, 1, N, N, 4, &ssw) ||
        !span_of(bias, bias ? 1 : 0, N, N, 4, &sb) || !span_of(Y, M, N, ldy, esy, &sy) ||
        !span_of(Z, Z ? M : 0, N, ldz, 4, &sz))
        return fail(MPDT_ERROR_INVALID_VALUE, fn, "operand too large");
    const Span ins[5] = {sx, sw, ssx, ssw, sb};
    for (const Span& in : ins)
        if (sy.overlaps(in) || sz.overlaps(in))
            return fail(MPDT_ERROR_ALIASING, fn, "an output overlaps an input");
    if (sy.overlaps(sz)) return fail(MPDT_ERROR_ALIASING, fn, "the output overlaps Z");
    mpdt_status s = check_device(fn);
    if (s != MPDT_SUCCESS) return s;
    mpdt::W8A8Args a{};
    a.X = X;
    a.ldx = ldx;
    a.x_scale = x_scale;
    a.W = W;
    a.ldw = ldw;
    a.w_scale = w_scale;
    a.bias = bias;
    if (requant) {
        a.Q = (int8_t*)Y;
        a.ldq = ldy;
        a.q_scale = out_scale;
    } else {
        a.Y = (uint16_t*)Y;
        a.ldy = ldy;
    }
    a.Z = Z;
    a.ldz = ldz;
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    a.w_kn = w_kn ? 1 : 0;
    const bool al = aligned_to(X, 16) && aligned_to(W, 16) && ldx % 16 == 0 && ldw % 16 == 0;
    return launched(mpdt::launch_gemm_w8a8(a, al, (hipStream_t)stream), fn);
}
}  // namespace

MPDT_EXPORT mpdt_status gemm_w8a8(int64_t M, int64_t N, int64_t K, const int8_t* X, int64_t ldx,
                                  const float* x_scale, const int8_t* W, int64_t ldw,
                                  const float* w_scale, const float* bias, uint16_t* Y, int64_t ldy,
                                  int32_t* Z, int64_t ldz, void* stream) {
    return run_w8a8("gemm_w8a8", M, N, K, X, ldx, x_scale, W, ldw, w_scale, bias, Y, ldy, false,
                    1.0f, Z, ldz, stream);
}

MPDT_EXPORT mpdt_status gemm_w8a8_kn(int64_t M, int64_t N, int64_t K, const int8_t* X, int64_t ldx,
                                     const float* x_scale, const int8_t* W, int64_t ldw,
                                     const float* w_scale, const float* bias, uint16_t* Y,
                                     int64_t ldy, int32_t* Z, int64_t ldz, void* stream) {
    return run_w8a8("gemm_w8a8_kn", M, N, K, X, ldx, x_scale, W, ldw, w_scale, bias, Y, ldy, false,
                    1.0f, Z, ldz, stream, true);
}

MPDT_EXPORT mpdt_status gemm_w8a8_requant(int64_t M, int64_t N, int64_t K, const int8_t* X,
                                          int64_t ldx, const float* x_scale, const int8_t* W,
                                          int64_t ldw, const float* w_scale, const float* bias,
                                          float out_scale, int8_t* Q, int64_t ldq, int32_t* Z,
                                          int64_t ldz, void* stream) {
    return run_w8a8("gemm_w8a8_requant", M, N, K, X, ldx, x_scale, W, ldw, w_scale, bias, Q, ldq,
                    true, out_scale, Z, ldz, stream);
}

MPDT_EXPORT mpdt_status quantize_i8_rows(int64_t M, int64_t K, const uint16_t* X, int64_t ldx,
                                         int8_t* Q, int64_t ldq, float* scales, void* stream) {
    const char* fn = "quantize_i8_rows";
    if (M < 0 || K < 0 || M > kMaxDim || K > kMaxDim)
        return fail(MPDT_ERROR_INVALID_VALUE, fn, "dimension out of range");
    if (M == 0) return MPDT_SUCCESS;
    if (!scales) return fail(MPDT_ERROR_INVALID_VALUE, fn, "scales is NULL");
    if (K > 0 && (!X || !Q)) return fail(MPDT_ERROR_INVALID_VALUE, fn, "X or Q is NULL");
    if (K > 0 && (ldx < K || ldq < K)) return fail(MPDT_ERROR_INVALID_VALUE, fn, "ldx or ldq < K");
    if ((X && !aligned_to(X, 2)) || !aligned_to(scales, 4))
        return fail(MPDT_ERROR_MISALIGNED, fn, "pointer not aligned to its element size");
    Span sx, sq, ss;
    if (!span_of(X, K > 0 ? M : 0, K, ldx, 2, &sx) || !span_of(Q, K > 0 ? M : 0, K, ldq, 1, &sq) ||
        !span_of(scales, 1, M, M, 4, &ss))
        return fail(MPDT_ERROR_INVALID_VALUE, fn, "operand too large");
    if (sq.overlaps(sx) || ss.overlaps(sx) || sq.overlaps(ss))
        return fail(MPDT_ERROR_ALIASING, fn, "an output overlaps the input or the other output");
    mpdt_status s = check_device(fn);
    if (s != MPDT_SUCCESS) return s;
    mpdt::QuantI8Args a{};
    a.X = X;
    a.ldx = ldx;
    a.Q = Q;
    a.ldq = ldq;
    a.S = scales;
    a.K = K;
    a.M = (int)M;
    a.vec = aligned_to(X, 16) && ldx % 8 == 0 && aligned_to(Q, 8) && ldq % 8 == 0;
    return launched(mpdt::launch_quantize_i8_rows(a, (hipStream_t)stream), fn);
}

namespace {
mpdt_status run_quantize_fp8(const char* fn, int64_t R, int64_t C, const float* X, int64_t ldx,
                             int fmt, int64_t br, int64_t bc, uint8_t* Q, int64_t ldq,
                             float* scales, int64_t lds, void* stream) {
    if (R < 0 || C < 0 || R > kMaxDim || C > kMaxDim)
        return fail(MPDT_ERROR_INVALID_VALUE, fn, "dimension out of range");
    if (fmt != MPDT_FP8_E4M3 && fmt != MPDT_FP8_E5M2)
        return fail(MPDT_ERROR_INVALID_VALUE, fn, "unknown FP8 format");
    if (br < 1 || bc < 1) return fail(MPDT_ERROR_INVALID_VALUE, fn, "block sizes must be positive");
    int shape;
    if (br >= R && bc >= C) shape = mpdt::FP8Q_TENSOR;
    else if (br == 1 && bc >= C) shape = mpdt::FP8Q_ROW;
    else if (bc == 1 && br >= R) shape = mpdt::FP8Q_COL;
    else if (br == 1 && bc == 128) shape = mpdt::FP8Q_ROW128;
    else if (br == 128 && bc == 128) shape = mpdt::FP8Q_TILE128;
    else return fail(MPDT_ERROR_INVALID_VALUE, fn, "unsupported block shape");
    if (R == 0 || C == 0) return MPDT_SUCCESS;
    const int64_t nbr = (R + br - 1) / br, nbc = (C + bc - 1) / bc;
    if (!X || !Q || !scales) return fail(MPDT_ERROR_INVALID_VALUE, fn, "X, Q or scales is NULL");
    if (ldx < C || ldq < C || lds < nbc)
        return fail(MPDT_ERROR_INVALID_VALUE, fn, "ldx or ldq < C, or lds < scale columns");
    if (!aligned_to(X, 4) || !aligned_to(scales, 4))
        return fail(MPDT_ERROR_MISALIGNED, fn, "pointer not aligned to its element size");
    Span sx, sq, ss;
    if (!span_of(X, R, C, ldx, 4, &sx) || !span_of(Q, R, C, ldq, 1, &sq) ||
        !span_of(scales, nbr, nbc, lds, 4, &ss))
        return fail(MPDT_ERROR_INVALID_VALUE, fn, "operand too large");
    if (sq.overlaps(sx) || ss.overlaps(sx) || sq.overlaps(ss))
        return fail(MPDT_ERROR_ALIASING, fn, "an output overlaps the input or the other output");
    mpdt_status s = check_device(fn);
    if (s != MPDT_SUCCESS) return s;
    mpdt::QuantFp8Args a{};
    a.X = X;
    a.ldx = ldx;
    a.Q = Q;
    a.ldq = ldq;
    a.S = scales;
    a.lds = lds;
    a.R = R;
    a.C = C;
    a.block_rows = (int)std::min<int64_t>(br, 128);
    a.fmt = fmt;
    a.shape = shape;
    a.vec = aligned_to(X, 16) && ldx % 4 == 0 && aligned_to(Q, 4) && ldq % 4 == 0;
    return launched(mpdt::launch_quantize_fp8_blocks(a, (hipStream_t)stream), fn);
}
}  // namespace

MPDT_EXPORT mpdt_status quantize_fp8_blocks(int64_t R, int64_t C, const float* X, int64_t ldx,
                                            int64_t block_rows, uint8_t* Q, int64_t ldq,
                                            float* scales, int64_t lds, void* stream) {
    const char* fn = "quantize_fp8_blocks";
    if (block_rows != 1 && block_rows != 128)
        return fail(MPDT_ERROR_INVALID_VALUE, fn, "block_rows must be 1 or 128");
    // (always the 1 x 128 / 128 x 128 kernels, whatever the matrix size)
    if (R < 0 || C < 0 || R > kMaxDim || C > kMaxDim)
        return fail(MPDT_ERROR_INVALID_VALUE, fn, "dimension out of range");
    if (R == 0 || C == 0) return MPDT_SUCCESS;
    const int64_t nbr = (R + block_rows - 1) / block_rows, nbc = (C + 127) / 128;
    if (!X || !Q || !scales) return fail(MPDT_ERROR_INVALID_VALUE, fn, "X, Q or scales is NULL");
    if (ldx < C || ldq < C || lds < nbc)
        return fail(MPDT_ERROR_INVALID_VALUE, fn, "ldx or ldq < C, or lds < ceil(C/128)");
    if (!aligned_to(X, 4) || !aligned_to(scales, 4))
        return fail(MPDT_ERROR_MISALIGNED, fn, "pointer not aligned to its element size");
    Span sx, sq, ss;
    if (!span_of(X, R, C, ldx, 4, &sx) || !span_of(Q, R, C, ldq, 1, &sq) ||
        !span_of(scales, nbr, nbc, lds, 4, &ss))
        return fail(MPDT_ERROR_INVALID_VALUE, fn, "operand too large");
    if (sq.overlaps(sx) || ss.overlaps(sx) || sq.overlaps(ss))
        return fail(MPDT_ERROR_ALIASING, fn, "an output overlaps the input or the other output");
    mpdt_status s = check_device(fn);
    if (s != MPDT_SUCCESS) return s;
    mpdt::QuantFp8Args a{};
    a.X = X;
    a.ldx = ldx;
    a.Q = Q;
    a.ldq = ldq;
    a.S = scales;
    a.lds = lds;
    a.R = R;
    a.C = C;
    a.block_rows = (int)block_rows;
    a.fmt = 0;
    a.shape = block_rows == 1 ? mpdt::FP8Q_ROW128 : mpdt::FP8Q_TILE128;
    a.vec = aligned_to(X, 16) && ldx % 4 == 0 && aligned_to(Q, 4) && ldq % 4 == 0;
    return launched(mpdt::launch_quantize_fp8_blocks(a, (hipStream_t)stream), fn);
}

MPDT_EXPORT mpdt_status quantize_fp8(int64_t R, int64_t C, const float* X, int64_t ldx, int fmt,
                                     int64_t block_rows, int64_t block_cols, uint8_t* Q, int64_t ldq,
                                     float* scales, int64_t lds, void* stream) {
    return run_quantize_fp8("quantize_fp8", R, C, X, ldx, fmt, block_rows, block_cols, Q, ldq, scales,
                            lds, stream);
}

MPDT_EXPORT const char* mpdt_status_string(mpdt_status s) {
    switch (s) {
        case MPDT_SUCCESS: return "success";
        case MPDT_ERROR_INVALID_VALUE: return "invalid value";
        case MPDT_ERROR_MISALIGNED: return "misaligned pointer";
        case MPDT_ERROR_ALIASING: return "output aliases an input";
        case MPDT_ERROR_NO_DEVICE: return "no HIP device";
        case MPDT_ERROR_UNSUPPORTED_DEVICE: return "unsupported device (gfx950 required)";
        case MPDT_ERROR_LAUNCH: return "kernel launch failed";
    }
    return "unknown status";
}

MPDT_EXPORT const char* mpdt_last_error(void) { return g_last_error.c_str(); }

MPDT_EXPORT int mpdt_version(void) { return 100; }
