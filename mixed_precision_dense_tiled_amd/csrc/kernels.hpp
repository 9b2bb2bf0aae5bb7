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
    const float* bias;    // fused epilogue: FP32 bias per output column (may be null)
    int act;              // fused epilogue: one of the ACT_* activations
    int fp8_fmt;          // FP8: bit 0 A is E5M2, bit 1 B is E5M2 (else E4M3)
    int row_scaled;       // FP8: sA / sB are per-row / per-column vectors, ld_sa /
                          // ld_sb their increments (0: one scale per tensor)
};

// The F8_* bits of an FP8 call (format of each operand, scaling variant).
inline int fp8_variant(const GemmArgs& a) { return (a.fp8_fmt & 3) | (a.row_scaled ? 4 : 0); }

// Activations of the fused epilogue (the values of the C ABI's mpdt_act).
enum : int { ACT_NONE = 0, ACT_RELU = 1, ACT_GELU = 2, ACT_SILU = 3 };

// aligned: every row start of A and B is 16-byte aligned.
hipError_t launch_gemm(Kind kind, const GemmArgs& a, bool aligned, hipStream_t stream);
// The FP8 GEMMs (gemm_fp8_general.hip): every tile of an eligible problem
// (or its full tiles only) on the one-wave kernel, the rest on the general
// kernel.
hipError_t launch_fp8(const GemmArgs& a, bool aligned, hipStream_t stream);
// FP16 / BF16 with the fused bias / activation epilogue (gemm_epi.hip).
hipError_t launch_gemm_epi(Kind kind, const GemmArgs& a, bool aligned, hipStream_t stream);

// FP8 one-wavefront kernel (gemm_fp8.hip) over the FP8_TILE_M x FP8_TILE_N
// tiles of a problem it takes.  fp8_1w_mode: 0 -- not at all; 1 -- its full
// tiles only; 2 -- every tile, edge tiles included (M >= FP8_TILE_M and N a
// multiple of 16 besides what mode 1 needs).
constexpr int FP8_TILE_M = 128, FP8_TILE_N = 256;
int fp8_1w_mode(const GemmArgs& a, bool aligned);
hipError_t launch_fp8_1w(const GemmArgs& a, int tiles_m, int tiles_n, hipStream_t stream);

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

// M-token W8A8 layer (M >= 1 tokens, per-token activation scales, optional
// bias).  Leading dimensions in elements.
struct W8A8Args {
    const int8_t* X;
    int64_t ldx;
    const float* x_scale;   // [M]
    const int8_t* W;
    int64_t ldw;
    const float* w_scale;   // [N]
    const float* bias;      // [N] or null
    uint16_t* Y;            // BF16 output, or null when Q is written
    int64_t ldy;
    int8_t* Q;              // INT8 requantised output (or null)
    int64_t ldq;
    float q_scale;          // Q = clamp(rne(value / q_scale), -127, 127)
    int32_t* Z;             // or null
    int64_t ldz;
    int M, N, K;
    int w_kn;               // W stored K x N (ldw >= N) instead of N x K
};

// aligned: X, W and their rows start 16-byte aligned.
hipError_t launch_gemm_w8a8(const W8A8Args& a, bool aligned, hipStream_t stream);

// Per-token INT8 quantisation of BF16 activations (M x K, leading dims in elements).
struct QuantI8Args {
    const uint16_t* X;
    int64_t ldx;
    int8_t* Q;
    int64_t ldq;
    float* S;
    int64_t K;
    int M;
    int vec;          // X rows 16-byte and Q rows 8-byte aligned: 8 elements per access
};
hipError_t launch_quantize_i8_rows(const QuantI8Args& a, hipStream_t stream);

// FP8 E4M3 block quantisation of an R x C FP32 matrix in block_rows x 128 blocks.
struct QuantFp8Args {
    const float* X;
    int64_t ldx;
    uint8_t* Q;
    int64_t ldq;
    float* S;
    int64_t lds;
    int64_t R, C;
    int block_rows;   // 1 or 128 (with 128 columns); or the shapes below
    int fmt;          // 0 E4M3, 1 E5M2
    int shape;        // FP8Q_* block shape
    int vec;          // X rows 16-byte and Q rows 4-byte aligned: 4 elements per access
};
// Block shapes of the FP8 quantiser: 1 x 128, 128 x 128, one scale per row
// (1 x C), per column (R x 1) or per tensor (R x C).
enum : int { FP8Q_ROW128 = 0, FP8Q_TILE128 = 1, FP8Q_ROW = 2, FP8Q_COL = 3, FP8Q_TENSOR = 4 };
hipError_t launch_quantize_fp8_blocks(const QuantFp8Args& a, hipStream_t stream);

}  // namespace mpdt
