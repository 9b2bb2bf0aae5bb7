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
// epilogue).
//   z[m][o] = sum_k X[m][k] * W[o][k]          (INT32, exact)
//   y[m][o] = bf16_rne( ((float(z) * s_x[m]) * s_w[o]) + bias[o] )
// or, requantised for a next layer that takes INT8 (same section),
//   q[m][o] = clamp(rne(( ... + bias[o]) / s_out), -127, 127)
// With more than one token the products are a small GEMM, Z = X . W^T, whose
// operands are both K-contiguous: a 32x32x32 INT8 MFMA takes 32 tokens
// (rows of X, zero past M) as its A operand and 32 output channels (rows of
// W) as its B operand, each lane reading 16 consecutive K bytes of one row
// straight from memory -- no LDS, no transposes.  The weights are streamed
// exactly once per 32 tokens: a workgroup owns 32 channels, its four waves
// take interleaved 128-byte slices of K (4 MFMA steps each, so every wave
// load covers 128 contiguous bytes of each of its 32 rows), then add their
// partial sums through LDS.  The work stays HBM-bound: the MFMA rate is far
// above what 32 tokens need, so the rows of the A operand past M cost nothing
// that matters.
// ---------------------------------------------------------------------------
constexpr int TOK_WAVES = 4;                   // wavefronts per workgroup
constexpr int TOK_GROUP = 8;                   // MFMA steps (32 K bytes each) per wave slice

__global__ __launch_bounds__(64 * TOK_WAVES) void gemm_w8a8_kernel(W8A8Args g) {
    __shared__ int partial[TOK_WAVES - 1][16][64];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int o0 = blockIdx.x * 32;
    const int r32 = lane & 31;                 // token row (A) / channel (B) of this lane
    const int half = lane >> 5;                // which 16 bytes of a 32-byte K step
    const int64_t K = g.K;
    const int64_t kslice = 32 * TOK_GROUP;     // K bytes per wave slice

    // this lane's rows: token r32 of X, channel o0 + r32 of W; a lane past M
    // or N reads row 0 instead and zeroes what it read, so the loads of a full
    // slice carry no branches (and stay in flight together)
    const bool xrow = r32 < g.M;
    const bool wrow = o0 + r32 < g.N;
    const char* xp = (const char*)g.X + (int64_t)(xrow ? r32 : 0) * g.ldx;
    const char* wp = (const char*)g.W + (int64_t)(wrow ? o0 + r32 : 0) * g.ldw;
    const uint32_t xkeep = xrow ? ~0u : 0u, wkeep = wrow ? ~0u : 0u;

    i32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0;
    auto mma = [&](const u32x4 (&xv)[TOK_GROUP], const u32x4 (&wv)[TOK_GROUP]) {
#pragma unroll
        for (int s = 0; s < TOK_GROUP; ++s)
            acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, xv[s]),
                                                        __builtin_bit_cast(i32x4, wv[s]), acc, 0, 0, 0);
    };
    int64_t k0 = (int64_t)wave * kslice;
    // full slices: plain 16-byte loads (any byte alignment is fine for them)
    for (; k0 + kslice <= K; k0 += (int64_t)TOK_WAVES * kslice) {
        u32x4 wv[TOK_GROUP], xv[TOK_GROUP];
#pragma unroll
        for (int s = 0; s < TOK_GROUP; ++s) {
            const int64_t off = k0 + 32 * s + 16 * half;
            wv[s] = *reinterpret_cast<const u32x4*>(wp + off) & wkeep;
            xv[s] = *reinterpret_cast<const u32x4*>(xp + off) & xkeep;
        }
        mma(xv, wv);
    }
    // the one partial slice (K past it reads as zero; bounded loads)
    if (k0 < K) {
        u32x4 wv[TOK_GROUP], xv[TOK_GROUP];
#pragma unroll
        for (int s = 0; s < TOK_GROUP; ++s) {
            const int64_t off = k0 + 32 * s + 16 * half;
            wv[s] = load16_row<false>(wp + off, wp + K) & wkeep;
            xv[s] = load16_row<false>(xp + off, xp + K) & xkeep;
        }
        mma(xv, wv);
    }

    // sum the four waves' partial products (exact INT32)
    if (wave > 0) {
#pragma unroll
        for (int r = 0; r < 16; ++r) partial[wave - 1][r][lane] = acc[r];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int w = 0; w < TOK_WAVES - 1; ++w)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] += partial[w][r][lane];

    // accumulator r of lane l: token 8 (r / 4) + 4 (l / 32) + r % 4, channel o0 + l % 32
    const int o = o0 + r32;
    if (o >= g.N) return;
    const float sw = g.w_scale[o];
    const float b = g.bias ? g.bias[o] : 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int m = 8 * (r >> 2) + 4 * half + (r & 3);
        if (m < g.M) {
            const int z = acc[r];
            if (g.Z) g.Z[(int64_t)m * g.ldz + o] = z;
            // three separately rounded FP32 operations (no fused multiply-add)
            float v = mul_rn((float)z, g.x_scale[m]);
            v = mul_rn(v, sw);
            if (g.bias) v = add_rn(v, b);
            if (g.Q) {
                // requantised for a next layer that takes INT8: one IEEE
                // division, round half to even, saturate to +-127
                const float q = __builtin_rintf(v / g.q_scale);
                g.Q[(int64_t)m * g.ldq + o] = (int8_t)fminf(fmaxf(q, -127.0f), 127.0f);
            } else {
                g.Y[(int64_t)m * g.ldy + o] = f32_to_bf16_bits(v);
            }
        }
    }
}

hipError_t launch_gemm_w8a8(const W8A8Args& a0, bool /*aligned*/, hipStream_t stream) {
    if (a0.N <= 0 || a0.M <= 0) return hipSuccess;
    // groups of at most 32 tokens, each group one launch reading W once
    for (int m0 = 0; m0 < a0.M; m0 += 32) {
        W8A8Args a = a0;
        a.M = min(32, a0.M - m0);
        a.X = a0.X + (int64_t)m0 * a0.ldx;
        a.x_scale = a0.x_scale + m0;
        a.Y = a0.Y ? a0.Y + (int64_t)m0 * a0.ldy : nullptr;
        a.Q = a0.Q ? a0.Q + (int64_t)m0 * a0.ldq : nullptr;
        a.Z = a0.Z ? a0.Z + (int64_t)m0 * a0.ldz : nullptr;
        dim3 grid((unsigned)((a.N + 31) / 32)), block(64 * TOK_WAVES);
        hipLaunchKernelGGL(gemm_w8a8_kernel, grid, block, 0, stream, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace mpdt
