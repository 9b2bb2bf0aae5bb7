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

// The epilogue of one 32-token x 32-channel block: accumulator r of lane l
// holds token 8 (r / 4) + 4 (l / 32) + r % 4 and channel o (= o0 + l % 32).
__device__ __forceinline__ void w8a8_epilogue(const W8A8Args& g, const i32x16& acc, int o, int half) {
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

    w8a8_epilogue(g, acc, o0 + r32, half);
}

// ---------------------------------------------------------------------------
// The same layer with the weights stored K x N (row k holds input k of every
// output channel, leading dimension ldw >= N): the logical [K][N] operand of
// x . W, for callers that keep weights that way.  The MFMA still needs 16
// consecutive K bytes of one channel per lane, so W is transposed through
// LDS.  A workgroup of four waves owns 64 channels and walks K in chunks of
// 1024 rows (64 KiB: each thread loads the 16-byte pieces of four
// consecutive rows in each of four 256-row blocks, with plain loads and no
// branches except in the last chunk and the last channel block, so all of
// them are in flight together).  Two register sets keep the loads of the
// next two chunks in flight while one is computed.  A chunk is written to
// LDS channel-major, four K bytes of one channel per 32-bit store (a byte
// transpose by v_perm; rows padded and swizzled so neither the stores nor
// the 16-byte operand reads have bank conflicts).  Wave w takes rows
// 256 w .. 256 w + 255 of every chunk (eight 32-K steps for each of the two
// 32-channel groups); the four partial sums meet in LDS as above.  The
// weights arrive as 64-byte pieces of many rows rather than long runs, and
// stream at about two thirds of the N x K layout's rate.
// ---------------------------------------------------------------------------
constexpr int KN_CH = 64;                       // channels per workgroup
constexpr int KN_PPR = KN_CH / 16;              // 16-byte pieces per row
constexpr int KN_RB = 4 * (256 / KN_PPR);       // rows per block (every thread: 4 rows x 1 piece)
constexpr int KN_NB = 4;                        // blocks per chunk
constexpr int KN_KC = KN_NB * KN_RB;            // K rows per chunk
constexpr int KN_KW = KN_KC / TOK_WAVES;        // rows of a chunk per wave
constexpr int KN_G = KN_CH / 32;                // 32-channel MFMA groups
// LDS: channel c's K bytes at c * KN_PITCH, K offset k stored at k ^ kn_swz(c).
constexpr int KN_PITCH = KN_KC + 16;
__device__ __forceinline__ int kn_swz(int c) { return (256 / KN_PPR) * ((c >> 4) & (KN_PPR - 1)); }

__global__ __launch_bounds__(256) void gemm_w8a8_kn_kernel(W8A8Args g) {
    __shared__ __attribute__((aligned(16))) uint8_t wt[2][KN_CH * KN_PITCH];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // Workgroups are dealt to the eight XCDs in turn; the channel blocks are
    // dealt so that each XCD gets one contiguous run of them.
    const int nblk = (g.N + KN_CH - 1) / KN_CH;
    const int per_xcd = (nblk + 7) / 8;
    const int blk = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    if (blk >= nblk) return;                     // whole workgroup: before any barrier
    const int o0 = blk * KN_CH;
    const int r32 = lane & 31, half = lane >> 5;
    const int64_t K = g.K;
    const int nch = (int)((K + KN_KC - 1) / KN_KC);
    // this thread's loads: rows KN_RB b + 4 (tid / KN_PPR) + i (b < KN_NB,
    // i < 4) of a chunk, bytes 16 (tid % KN_PPR) .. +15 of the workgroup's
    // channel piece (bounded by N: bytes past it read as zero)
    const int lg = tid / KN_PPR, lc = (tid % KN_PPR) * 16;
    const char* const wbase = (const char*)g.W + o0 + lc;
    const int64_t wlen = (int64_t)g.N - o0 - lc;          // valid bytes of the piece
    const int64_t wend = wlen < 16 ? (wlen > 0 ? wlen : 0) : 16;
    // Whole chunks of whole pieces take plain 16-byte loads (any byte address
    // is fine for them) with no branches, so all 16 stay in flight together;
    // the last chunk and the last channel block take the bounded loads.
    const bool full_n = o0 + KN_CH <= g.N;
    auto load_chunk = [&](int c, u32x4 (&v)[KN_NB][4]) {
        const int64_t k0 = (int64_t)c * KN_KC + 4 * lg;
        if (full_n && (int64_t)(c + 1) * KN_KC <= K) {
            const char* p = wbase + k0 * g.ldw;
#pragma unroll
            for (int b = 0; b < KN_NB; ++b)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    v[b][i] = *reinterpret_cast<const u32x4*>(p + (int64_t)(KN_RB * b + i) * g.ldw);
        } else {
#pragma unroll
            for (int b = 0; b < KN_NB; ++b)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int64_t k = k0 + KN_RB * b + i;
                    const char* p = wbase + k * g.ldw;
                    v[b][i] = (k < K) ? load16_row<false>(p, p + wend) : u32x4{0u, 0u, 0u, 0u};
                }
        }
    };
    // channel lc + q, K bytes KN_RB b + 4 lg .. +3 of the chunk: byte q of
    // the four rows' pieces, as one 32-bit LDS store
    auto store_chunk = [&](int buf, const u32x4 (&v)[KN_NB][4]) {
#pragma unroll
        for (int b = 0; b < KN_NB; ++b)
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                // byte q of the four rows' pieces: two byte pairs, then the word
                // (v_perm: selector bytes 0-3 pick the second operand, 4-7 the first)
                const int w = q >> 2;
                const uint32_t sel = 0x0c0c0400u | (uint32_t)(q & 3) | ((uint32_t)(q & 3) << 8);
                const uint32_t lo = __builtin_amdgcn_perm(v[b][1][w], v[b][0][w], sel);
                const uint32_t hi = __builtin_amdgcn_perm(v[b][3][w], v[b][2][w], sel);
                const uint32_t word = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
                const int ch = lc + q;
                *reinterpret_cast<uint32_t*>(&wt[buf][ch * KN_PITCH + ((KN_RB * b + 4 * lg) ^ kn_swz(ch))]) = word;
            }
    };
    const bool xrow = r32 < g.M;
    const char* xp = (const char*)g.X + (int64_t)(xrow ? r32 : 0) * g.ldx;
    const uint32_t xkeep = xrow ? ~0u : 0u;

    i32x16 acc[KN_G];
#pragma unroll
    for (int j = 0; j < KN_G; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][r] = 0;
    // Two register sets: the loads of chunks c + 1 and c + 2 are in flight
    // while chunk c is computed.
    u32x4 va[KN_NB][4], vb[KN_NB][4];
    load_chunk(0, va);
    if (nch > 1) load_chunk(1, vb);
    auto step = [&](int c, u32x4 (&v)[KN_NB][4]) {
        const int buf = c & 1;
        store_chunk(buf, v);
        __syncthreads();
        if (c + 2 < nch) load_chunk(c + 2, v);          // in flight during the MFMAs
        const int64_t kw = (int64_t)c * KN_KC + KN_KW * wave;
        constexpr int NS = KN_KW / 32;                  // 32-K steps per wave and chunk
        u32x4 xv[NS];
        if ((int64_t)(c + 1) * KN_KC <= K) {
#pragma unroll
            for (int s = 0; s < NS; ++s)
                xv[s] = *reinterpret_cast<const u32x4*>(xp + kw + 32 * s + 16 * half) & xkeep;
        } else {
#pragma unroll
            for (int s = 0; s < NS; ++s) xv[s] = load16_row<false>(xp + kw + 32 * s + 16 * half, xp + K) & xkeep;
        }
#pragma unroll
        for (int s = 0; s < NS; ++s) {
#pragma unroll
            for (int j = 0; j < KN_G; ++j) {
                // channel 32 j + r32, K bytes KN_KW wave + 32 s + 16 half .. +15 of the chunk
                const int ch = 32 * j + r32;
                const u32x4 wv = *reinterpret_cast<const u32x4*>(
                    &wt[buf][ch * KN_PITCH + ((KN_KW * wave + 32 * s + 16 * half) ^ kn_swz(ch))]);
                acc[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, xv[s]),
                                                               __builtin_bit_cast(i32x4, wv), acc[j], 0, 0, 0);
            }
        }
    };
    for (int c = 0; c < nch; c += 2) {
        step(c, va);
        if (c + 1 < nch) step(c + 1, vb);
    }
    // partial sums of waves 1..3 through the first chunk buffer, once every
    // wave is done reading it
    __syncthreads();
    int* const partial = reinterpret_cast<int*>(&wt[0][0]);   // [3][KN_G][16][64]
    static_assert((TOK_WAVES - 1) * KN_G * 16 * 64 * 4 <= KN_CH * KN_PITCH, "partial sums fit");
    if (wave > 0) {
#pragma unroll
        for (int j = 0; j < KN_G; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) partial[(((wave - 1) * KN_G + j) * 16 + r) * 64 + lane] = acc[j][r];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int j = 0; j < KN_G; ++j) {
#pragma unroll
        for (int w = 0; w < TOK_WAVES - 1; ++w)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[j][r] += partial[((w * KN_G + j) * 16 + r) * 64 + lane];
        w8a8_epilogue(g, acc[j], o0 + 32 * j + r32, half);
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
        if (a.w_kn) {
            const int nblk = (a.N + KN_CH - 1) / KN_CH;
            hipLaunchKernelGGL(gemm_w8a8_kn_kernel, dim3((unsigned)(8 * ((nblk + 7) / 8))), dim3(256), 0,
                               stream, a);
        } else {
            dim3 grid((unsigned)((a.N + 31) / 32)), block(64 * TOK_WAVES);
            hipLaunchKernelGGL(gemm_w8a8_kernel, grid, block, 0, stream, a);
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace mpdt
