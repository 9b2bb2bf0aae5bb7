// gemv_w8a8.hip -- batch-1 W8A8 linear layer for gfx950, a streaming
// wavefront-reduction kernel (no matrix instructions).
//
// The operation is the one of "NVIDIA A100: from chip to SIMT", sections 5.1
// and 5.2: z[o] = sum_k x[k] * W[o][k] with symmetric INT8 operands summed
// exactly in INT32, then y[o] = (float(z[o]) * s_x) * s_w[o] in the epilogue
// (rounded here to BF16), with W stored one output channel per row.  That
// page's teaching kernel pads the single activation row into 16-row matrix
// tiles (about 16x wasted arithmetic, section 5.5) and notes the layer is
// weight-bandwidth bound; this kernel instead streams W once at HBM rate:
//
//   * one wavefront owns R consecutive output rows; lane l reads the 16-byte
//     chunks l, l + 64, l + 128, ... of each row (every load instruction moves
//     1 KiB of one row, fully coalesced) and the matching chunks of x (4 KiB,
//     shared by all waves through L2);
//   * all R * (K / 1024) loads of a wave are issued before the first use, so
//     a resident grid keeps the whole weight stream in flight (R = 2 keeps
//     the register count at 72, seven waves per SIMD: the 14336-row layer
//     fits the chip in one round);
//   * v_dot4 accumulates 4 byte products per instruction into INT32;
//   * a butterfly over the 64 lanes reduces each row; lane r writes row r.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.hpp"
#include "kernels.hpp"

namespace mpdt {

constexpr int GEMV_WAVES = 4;        // wavefronts per workgroup
constexpr int GEMV_ROWS = 2;         // output rows per wavefront (72 VGPRs: 7 waves per SIMD,
                                     // so the whole 14336-row layer is resident at once)
constexpr int GEMV_U = 4;            // 16-byte chunks per lane per row per pass (K = 4096 in one pass)

__device__ __forceinline__ int dot16(u32x4 w, u32x4 x, int acc) {
#pragma unroll
    for (int q = 0; q < 4; ++q) acc = __builtin_amdgcn_sdot4((int)w[q], (int)x[q], acc, false);
    return acc;
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

template <bool ALIGNED>
__global__ __launch_bounds__(64 * GEMV_WAVES) void gemv_w8a8_kernel(GemvArgs g) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int row0 = (blockIdx.x * GEMV_WAVES + wave) * GEMV_ROWS;
    if (row0 >= g.N) return;                      // whole wave past the end: nothing to do

    const int64_t kbytes = g.K;
    const char* x = (const char*)g.x;
    const char* xend = x + kbytes;
    int acc[GEMV_ROWS];
#pragma unroll
    for (int r = 0; r < GEMV_ROWS; ++r) acc[r] = 0;

    for (int64_t kb = 0; kb < kbytes; kb += 64 * 16 * GEMV_U) {
        u32x4 xv[GEMV_U];
        u32x4 wv[GEMV_ROWS][GEMV_U];
#pragma unroll
        for (int u = 0; u < GEMV_U; ++u) {
            const int64_t off = kb + 16 * (lane + 64 * u);
            xv[u] = (ALIGNED && off + 16 <= kbytes) ? load16_fast(x + off)
                                                     : load16_row<ALIGNED>(x + off, xend);
        }
#pragma unroll
        for (int r = 0; r < GEMV_ROWS; ++r) {
            const int row = row0 + r;
            const char* rowp = (const char*)g.W + (int64_t)row * g.ldw;
#pragma unroll
            for (int u = 0; u < GEMV_U; ++u) {
                const int64_t off = kb + 16 * (lane + 64 * u);
                const char* p = rowp + off;
                if (row >= g.N)
                    wv[r][u] = u32x4{0u, 0u, 0u, 0u};
                else if (ALIGNED && off + 16 <= kbytes)
                    // streamed once: non-temporal, so it does not displace x in the caches
                    wv[r][u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
                else
                    wv[r][u] = load16_row<ALIGNED>(p, rowp + kbytes);
            }
        }
#pragma unroll
        for (int r = 0; r < GEMV_ROWS; ++r)
#pragma unroll
            for (int u = 0; u < GEMV_U; ++u) acc[r] = dot16(wv[r][u], xv[u], acc[r]);
    }

    int z[GEMV_ROWS];
#pragma unroll
    for (int r = 0; r < GEMV_ROWS; ++r) z[r] = wave_sum(acc[r]);

#pragma unroll
    for (int r = 0; r < GEMV_ROWS; ++r) {
        const int row = row0 + r;
        if (lane == r && row < g.N) {
            if (g.z) g.z[row] = z[r];
            // dequantise: two FP32 products, activation scale first
            float v = (float)z[r];
            v = v * g.x_scale;
            v = v * g.w_scale[row];
            g.y[row] = f32_to_bf16_bits(v);
        }
    }
}

hipError_t launch_gemv_w8a8(const GemvArgs& a, bool aligned, hipStream_t stream) {
    if (a.N <= 0) return hipSuccess;
    const int rows_per_wg = GEMV_WAVES * GEMV_ROWS;
    dim3 grid((unsigned)((a.N + rows_per_wg - 1) / rows_per_wg)), block(64 * GEMV_WAVES);
    if (aligned)
        hipLaunchKernelGGL(gemv_w8a8_kernel<true>, grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL(gemv_w8a8_kernel<false>, grid, block, 0, stream, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// The same layer for M tokens at once (a small batch), each with its own
// activation scale, and an optional bias added after the dequantisation
// (section 5.1 of the same page: a bias belongs in the floating-point
// epilogue).  The weights are still streamed from HBM exactly once for up to
// 16 tokens: the workgroup stages the tokens' K slice in LDS, each wave owns
// two output channels and, for every 16-byte chunk of a weight row, takes the
// v_dot4 products with the same chunk of every token.  Larger batches are cut
// into groups of 16 tokens on the host (one launch each).
//   z[m][o] = sum_k X[m][k] * W[o][k]          (INT32, exact)
//   y[m][o] = bf16_rne( ((float(z) * s_x[m]) * s_w[o]) + bias[o] )
// ---------------------------------------------------------------------------
constexpr int TOK_WAVES = 4;       // wavefronts per workgroup
constexpr int TOK_ROWS = 2;        // output channels per wavefront
constexpr int TOK_KC = 4096;       // K bytes staged per pass (MG * 4 KiB of LDS)

template <int MG, bool ALIGNED>
__global__ __launch_bounds__(64 * TOK_WAVES) void gemm_w8a8_kernel(W8A8Args g) {
    __shared__ __attribute__((aligned(16))) char xs[MG][TOK_KC];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int row0 = (blockIdx.x * TOK_WAVES + wave) * TOK_ROWS;
    const int64_t K = g.K;

    int acc[TOK_ROWS][MG];
#pragma unroll
    for (int r = 0; r < TOK_ROWS; ++r)
#pragma unroll
        for (int m = 0; m < MG; ++m) acc[r][m] = 0;

    for (int64_t kc = 0; kc < K; kc += TOK_KC) {
        const int64_t kn = min((int64_t)TOK_KC, K - kc);   // valid bytes of this pass
        // stage the tokens' K slice (zero past M and past K)
        for (int i = tid; i < MG * (TOK_KC / 16); i += 64 * TOK_WAVES) {
            const int m = i / (TOK_KC / 16), c = i % (TOK_KC / 16);
            u32x4 v = u32x4{0u, 0u, 0u, 0u};
            if (m < g.M) {
                const char* rowp = (const char*)g.X + (int64_t)m * g.ldx + kc;
                v = load16_row<ALIGNED>(rowp + c * 16, rowp + kn);
            }
            lds_store16(lds_cast(xs[m]), c * 16, v);
        }
        __syncthreads();
        // weights of this wave's rows for the whole pass, then the products
        u32x4 wv[TOK_ROWS][TOK_KC / 1024];
#pragma unroll
        for (int r = 0; r < TOK_ROWS; ++r) {
            const int row = row0 + r;
            const char* rowp = (const char*)g.W + (int64_t)row * g.ldw + kc;
#pragma unroll
            for (int u = 0; u < TOK_KC / 1024; ++u) {
                const int64_t off = 16 * (lane + 64 * u);
                if (row >= g.N)
                    wv[r][u] = u32x4{0u, 0u, 0u, 0u};
                else if (ALIGNED && off + 16 <= kn)
                    wv[r][u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(rowp + off));
                else
                    wv[r][u] = load16_row<ALIGNED>(rowp + off, rowp + kn);
            }
        }
#pragma unroll
        for (int u = 0; u < TOK_KC / 1024; ++u) {
#pragma unroll
            for (int m = 0; m < MG; ++m) {
                const u32x4 xv = lds_load16(lds_cast(xs[m]), (uint32_t)(16 * (lane + 64 * u)));
#pragma unroll
                for (int r = 0; r < TOK_ROWS; ++r) acc[r][m] = dot16(wv[r][u], xv, acc[r][m]);
            }
        }
        __syncthreads();
    }

#pragma unroll
    for (int r = 0; r < TOK_ROWS; ++r)
#pragma unroll
        for (int m = 0; m < MG; ++m) acc[r][m] = wave_sum(acc[r][m]);

    // lane r * MG + m writes channel row0 + r of token m
#pragma unroll
    for (int r = 0; r < TOK_ROWS; ++r)
#pragma unroll
        for (int m = 0; m < MG; ++m) {
            const int row = row0 + r;
            if (lane == r * MG + m && row < g.N && m < g.M) {
                const int z = acc[r][m];
                if (g.Z) g.Z[(int64_t)m * g.ldz + row] = z;
                float v = (float)z;
                v = v * g.x_scale[m];
                v = v * g.w_scale[row];
                if (g.bias) v = v + g.bias[row];
                g.Y[(int64_t)m * g.ldy + row] = f32_to_bf16_bits(v);
            }
        }
}

template <int MG>
static hipError_t launch_tokens(const W8A8Args& a, bool aligned, hipStream_t stream) {
    const int rows_per_wg = TOK_WAVES * TOK_ROWS;
    dim3 grid((unsigned)((a.N + rows_per_wg - 1) / rows_per_wg)), block(64 * TOK_WAVES);
    if (aligned)
        hipLaunchKernelGGL((gemm_w8a8_kernel<MG, true>), grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((gemm_w8a8_kernel<MG, false>), grid, block, 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_gemm_w8a8(const W8A8Args& a0, bool aligned, hipStream_t stream) {
    if (a0.N <= 0 || a0.M <= 0) return hipSuccess;
    // groups of at most 16 tokens, each group one launch reading W once
    for (int m0 = 0; m0 < a0.M; m0 += 16) {
        W8A8Args a = a0;
        a.M = min(16, a0.M - m0);
        a.X = a0.X + (int64_t)m0 * a0.ldx;
        a.x_scale = a0.x_scale + m0;
        a.Y = a0.Y + (int64_t)m0 * a0.ldy;
        a.Z = a0.Z ? a0.Z + (int64_t)m0 * a0.ldz : nullptr;
        hipError_t e;
        if (a.M == 1) e = launch_tokens<1>(a, aligned, stream);
        else if (a.M == 2) e = launch_tokens<2>(a, aligned, stream);
        else if (a.M <= 4) e = launch_tokens<4>(a, aligned, stream);
        else if (a.M <= 8) e = launch_tokens<8>(a, aligned, stream);
        else e = launch_tokens<16>(a, aligned, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace mpdt
