// kernels.hpp -- internal (C++) interface between the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mpdt {

enum class Kind { F16, BF16, I8, FP8 };

// Arguments of one GEMM launch.  Leading dimensions of A and B in BYTES, of
// C and D in elements.  For FP8, sA / sB are the block-scale grids.
struct GemmArgs {
    const char* A;
    const char* B;
    const void* C;
    void* D;
    int64_t lda_b, ldb_b, ldc, ldd;
    int M, N, K;
    const float* sA;
    int64_t ld_sa;
    const float* sB;
    int64_t ld_sb;
    int tiles_m, tiles_n;
    int int_tm, int_tn;   // interior tiles launched separately (0: none)
    int out16;            // FP16/BF16 inputs: D is written in the input format (RNE)
    int d16_vec;          // out16 with D and its rows 16-byte aligned: wide stores allowed
};

// aligned: every row start of A and B is 16-byte aligned.
hipError_t launch_gemm(Kind kind, const GemmArgs& a, bool aligned, hipStream_t stream);

struct GemvArgs {
    const int8_t* x;
    const int8_t* W;
    int64_t ldw;
    const float* w_scale;
    uint16_t* y;
    int32_t* z;
    float x_scale;
    int N, K;
};

// aligned: x and every row of W start 16-byte aligned.
hipError_t launch_gemv_w8a8(const GemvArgs& a, bool aligned, hipStream_t stream);

}  // namespace mpdt
