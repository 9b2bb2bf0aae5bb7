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
//     the register count under 72, seven waves per SIMD: the 14336-row layer
//     fits the chip in one round, two 14-wave workgroups per CU);
//   * the rows' weight scales are requested before the weights, so no
//     memory round trip is left for the end of the wave;
//   * v_dot4 accumulates 4 byte products per instruction into INT32;
//   * DPP moves reduce each row over the 64 lanes; lane r writes row r.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.hpp"
#include "kernels.hpp"

namespace mpdt {

constexpr int GEMV_WAVES = 14;       // wavefronts per workgroup (896 threads; two workgroups
                                     // fill a CU at 7 waves per SIMD)
constexpr int GEMV_ROWS = 2;         // output rows per wavefront (<= 72 VGPRs: 7 waves per SIMD,
                                     // so the whole 14336-row layer is resident at once)
constexpr int GEMV_U = 4;            // 16-byte chunks per lane per row per pass (K = 4096 in one pass)

__device__ __forceinline__ int dot16(u32x4 w, u32x4 x, int acc) {
#pragma unroll
    for (int q = 0; q < 4; ++q) acc = __builtin_amdgcn_sdot4((int)w[q], (int)x[q], acc, false);
    return acc;
}

// Sum over the 64 lanes of a fully active wavefront, returned wave-uniform
// (scalar registers): DPP moves inside each row of 16 lanes (quad swaps, then
// the half-row and row mirrors), then the four row sums read into scalar
// registers.  No LDS round trip: a shuffle per step (ds_bpermute) costs an
// LDS latency each, six times over at the end of every wave.  Integer adds,
// so the order does not change the result.
__device__ __forceinline__ int wave_sum(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0xb1, 0xf, 0xf, false);    // quad_perm [1, 0, 3, 2]
    v += __builtin_amdgcn_update_dpp(0, v, 0x4e, 0xf, 0xf, false);    // quad_perm [2, 3, 0, 1]
    v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xf, 0xf, false);   // row_half_mirror
    v += __builtin_amdgcn_update_dpp(0, v, 0x140, 0xf, 0xf, false);   // row_mirror
    return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) +
           __builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48);
}

// FULL: x and every row of W are 16-byte aligned and K is a whole number of
// passes (K % 4096 == 0; the host checks it): no chunk is partial, so the
// loads of a pass carry no bounds, and the weight loads go out first.  The
// wave's rows past N (only in the last wave) still take the bounded form.
template <bool ALIGNED, bool FULL = false>
__global__ __launch_bounds__(64 * GEMV_WAVES) void gemv_w8a8_kernel(GemvArgs g) {
    static_assert(!FULL || ALIGNED, "whole passes need aligned rows");
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int row0 = (blockIdx.x * GEMV_WAVES + wave) * GEMV_ROWS;
    if (row0 >= g.N) return;                      // whole wave past the end: nothing to do
    // the rows' weight scales, requested before the weights (a row past N
    // reads row N - 1 and is not written): fetched after the reduction they
    // would add a memory round trip to the end of every wave.  (Relaxed
    // atomic loads, so the compiler does not sink them to their use.)
    float sw[GEMV_ROWS];
#pragma unroll
    for (int r = 0; r < GEMV_ROWS; ++r)
        sw[r] = __hip_atomic_load(&g.w_scale[min(row0 + r, g.N - 1)], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);

    const int64_t kbytes = g.K;
    const char* x = (const char*)g.x;
    const char* xend = x + kbytes;
    int acc[GEMV_ROWS];
#pragma unroll
    for (int r = 0; r < GEMV_ROWS; ++r) acc[r] = 0;

    if (FULL && row0 + GEMV_ROWS <= g.N) {
        for (int64_t kb = 0; kb < kbytes; kb += 64 * 16 * GEMV_U) {
            u32x4 wv[GEMV_ROWS][GEMV_U], xv[GEMV_U];
#pragma unroll
            for (int r = 0; r < GEMV_ROWS; ++r)
#pragma unroll
                for (int u = 0; u < GEMV_U; ++u)
                    wv[r][u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
                        (const char*)g.W + (int64_t)(row0 + r) * g.ldw + kb + 16 * (lane + 64 * u)));
#pragma unroll
            for (int u = 0; u < GEMV_U; ++u) xv[u] = load16_fast(x + kb + 16 * (lane + 64 * u));
#pragma unroll
            for (int r = 0; r < GEMV_ROWS; ++r)
#pragma unroll
                for (int u = 0; u < GEMV_U; ++u) acc[r] = dot16(wv[r][u], xv[u], acc[r]);
        }
    } else
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

    // lane r writes row r: one store instruction for all the wave's rows
    if (lane < GEMV_ROWS && row0 + lane < g.N) {
        int zr = z[0];
        float swr = sw[0];
#pragma unroll
        for (int r = 1; r < GEMV_ROWS; ++r) {
            if (lane == r) {
                zr = z[r];
                swr = sw[r];
            }
        }
        const int row = row0 + lane;
        if (g.z) g.z[row] = zr;
        // dequantise: two FP32 products, activation scale first
        float v = (float)zr;
        v = v * g.x_scale;
        v = v * swr;
        g.y[row] = f32_to_bf16_bits(v);
    }
}

hipError_t launch_gemv_w8a8(const GemvArgs& a, bool aligned, hipStream_t stream) {
    if (a.N <= 0) return hipSuccess;
    const int rows_per_wg = GEMV_WAVES * GEMV_ROWS;
    dim3 grid((unsigned)((a.N + rows_per_wg - 1) / rows_per_wg)), block(64 * GEMV_WAVES);
    if (aligned && a.K % (64 * 16 * GEMV_U) == 0)
        hipLaunchKernelGGL((gemv_w8a8_kernel<true, true>), grid, block, 0, stream, a);
    else if (aligned)
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
// (rows of X) as its A operand and 32 output channels (rows of W) as its B
// operand, each lane holding 16 consecutive K bytes of one row.  The weights
// are streamed exactly once per 32 tokens: a workgroup owns 32 channels and
// its four waves load them in long runs (one KiB of one row per load
// instruction, the access pattern of the one-token kernel; loading the MFMA
// fragments straight from memory instead touches 32 rows with 32 bytes each
// per instruction, and streamed about 7 % slower), staged through LDS
// chunk by chunk; wave w takes a quarter of each chunk's K bytes, and the
// four partial sums meet in LDS.  Up to 16 tokens their rows take the same
// road (one KiB of one row per load, staged beside the weights): loaded as
// per-lane fragments, 32 rows x 32 bytes per instruction, they took a sixth
// of the layer's time at 16 tokens.  The work stays HBM-bound: the
// MFMA rate is far above what 32 tokens need, so the rows of the A operand
// past M cost nothing that matters.
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
constexpr int TOK_CH = 32;                     // output channels per workgroup
constexpr int TOK_KC = 1024;                   // K bytes per LDS chunk
constexpr int TOK_PASS = 4;                    // chunks per pass (K = 4096 in one pass)
constexpr int TOK_PITCH = TOK_KC + 16;         // LDS row pitch: 16 bytes of padding per row

// XL (at most 16 tokens): token rows staged through LDS, each a contiguous
// KiB per chunk loaded once per workgroup; otherwise (at most 32 tokens; the
// staged form's registers would not fit) every lane loads its own MFMA
// fragments of the tokens (32 rows x 32 bytes per load instruction).
template <bool XL>
__global__ __launch_bounds__(64 * TOK_WAVES) __attribute__((amdgpu_waves_per_eu(2))) void gemm_w8a8_kernel(W8A8Args g) {
    // one chunk of the workgroup's 32 weight rows (then the partial sums),
    // and the same chunk of the token rows
    __shared__ __attribute__((aligned(16))) char wt[TOK_CH * TOK_PITCH];
    __shared__ __attribute__((aligned(16))) char xt[XL ? 16 * TOK_PITCH : 16];
    static_assert((TOK_WAVES - 1) * 16 * 64 * 4 <= TOK_CH * TOK_PITCH, "partial sums fit");
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int o0 = blockIdx.x * TOK_CH;
    const int r32 = lane & 31;                 // token row (A) / channel (B) of this lane
    const int half = lane >> 5;                // which 16 bytes of a 32-byte K step
    const int64_t K = g.K;
    constexpr int RPW = TOK_CH / TOK_WAVES;    // weight rows each wave loads
    constexpr int XPW = XL ? 16 / TOK_WAVES : 8;   // token rows each wave loads / fragments per lane
    MPDT_LDS char* const lds = lds_cast(wt);
    MPDT_LDS char* const xl = lds_cast(xt);

    // the rows this wave loads (a row past N reads row N - 1: its channel's
    // sums are never written)
    const char* wrow[RPW];
#pragma unroll
    for (int j = 0; j < RPW; ++j) {
        const int o = o0 + wave * RPW + j;
        wrow[j] = (const char*)g.W + (int64_t)(o < g.N ? o : g.N - 1) * g.ldw;
    }
    // XL: token rows wave, wave + 4, ... below M, each a contiguous KiB per
    // chunk, staged through LDS beside the weights; the MFMA's rows past M
    // read whatever the token buffer holds there (rows 16..31 read rows
    // 0..15 again).  Otherwise the token row of this lane (a row past M reads
    // row 0).  Only outputs past M see those rows, and none is written.
    const int xrows = g.M > wave ? (g.M - wave + TOK_WAVES - 1) / TOK_WAVES : 0;
    const char* const xp = (const char*)g.X + (int64_t)(r32 < g.M ? r32 : 0) * g.ldx;
    // Full passes read the weights and the tokens through buffer resources:
    // a row's offset goes in a scalar register and one lane offset serves
    // every load (64-bit per-row lane addresses would take 16 registers).
    const int row0 = o0 + wave * RPW;
    const __amdgpu_buffer_rsrc_t wrs = buffer_rsrc((const char*)g.W + (int64_t)min(row0, g.N - 1) * g.ldw, 0xffffffffu);
    const __amdgpu_buffer_rsrc_t xrs = buffer_rsrc((const char*)g.X + (int64_t)wave * g.ldx, 0xffffffffu);
    uint32_t wsoff[RPW];
#pragma unroll
    for (int j = 0; j < RPW; ++j)
        wsoff[j] = (uint32_t)((int64_t)(min(row0 + j, g.N - 1) - min(row0, g.N - 1)) * g.ldw);
    const uint32_t lane16 = 16u * (uint32_t)lane;
    // (the lane and scalar offsets are added in 32 bits: passes take this
    // path only while the largest sums stay below 2^32)
    const bool wbuf = (int64_t)(RPW - 1) * g.ldw + K + 4096 < (int64_t(1) << 32) &&
                      (int64_t)(16 - TOK_WAVES) * g.ldx + K + 4096 < (int64_t(1) << 32);

    i32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0;

    // Passes of TOK_PASS chunks.  Each wave first issues the loads of its
    // rows for the whole pass -- every instruction one contiguous KiB of one
    // row, as in the one-token kernel, so a resident grid keeps the weight
    // stream in flight -- then, chunk by chunk, the workgroup writes the
    // chunk's weight and token rows to LDS and wave w takes its K bytes
    // 256 w .. 256 w + 255 in eight MFMA steps (operands: 16 bytes of one
    // token and 16 bytes of one channel, both from LDS).  A pass inside K
    // takes plain 16-byte loads (any byte alignment is fine for them); the
    // last, partial one bounded loads (bytes past K read as zero).
    for (int64_t p0 = 0; p0 < K; p0 += (int64_t)TOK_PASS * TOK_KC) {
        const bool full = wbuf && p0 + (int64_t)TOK_PASS * TOK_KC <= K;
        auto load_x = [&](int c, u32x4 (&xr)[XPW]) {
            if constexpr (!XL) {
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    const int64_t off = p0 + c * TOK_KC + wave * 256 + 32 * s + 16 * half;
                    xr[s] = full ? *reinterpret_cast<const u32x4*>(xp + off) : load16_row<false>(xp + off, xp + K);
                }
                return;
            }
#pragma unroll
            for (int i = 0; i < XPW; ++i) {
                if (i < xrows) {
                    const int64_t off = p0 + c * TOK_KC;
                    if (full) {
                        xr[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                              xrs, (uint32_t)off + lane16,
                                                              (uint32_t)(TOK_WAVES * i) * (uint32_t)g.ldx, 0));
                    } else {
                        const char* xq = (const char*)g.X + (int64_t)(wave + TOK_WAVES * i) * g.ldx;
                        xr[i] = load16_row<false>(xq + off + lane16, xq + K);
                    }
                }
            }
        };
        // write chunk c of this wave's weight and token rows to LDS, then
        // its eight MFMA steps
        auto chunk = [&](int c, const u32x4 (&w)[RPW], const u32x4 (&xr)[XPW]) {
            __syncthreads();                       // the previous chunk's reads are done
#pragma unroll
            for (int j = 0; j < RPW; ++j)
                lds_store16(lds, (uint32_t)((wave * RPW + j) * TOK_PITCH + 16 * lane), w[j]);
            if constexpr (XL) {
#pragma unroll
                for (int i = 0; i < XPW; ++i)
                    if (i < xrows) lds_store16(xl, (uint32_t)((wave + TOK_WAVES * i) * TOK_PITCH + 16 * lane), xr[i]);
            }
            __syncthreads();
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const uint32_t ko = (uint32_t)(wave * 256 + 32 * s + 16 * half);
                const u32x4 a = XL ? lds_load16(xl, (uint32_t)((r32 & 15) * TOK_PITCH) + ko) : xr[s];
                const u32x4 b = lds_load16(lds, (uint32_t)(r32 * TOK_PITCH) + ko);
                acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, a),
                                                            __builtin_bit_cast(i32x4, b), acc, 0, 0, 0);
            }
        };
        auto load_w = [&](u32x4 (&wv)[TOK_PASS][RPW]) {
#pragma unroll
            for (int c = 0; c < TOK_PASS; ++c)
#pragma unroll
                for (int j = 0; j < RPW; ++j)
                    wv[c][j] = __builtin_bit_cast(
                        u32x4, __builtin_amdgcn_raw_buffer_load_b128(wrs, (uint32_t)p0 + c * TOK_KC + lane16, wsoff[j], 0));
        };
        static_assert(TOK_PASS == 4, "four chunks per pass");
        if (full && XL) {
            // Issue order: the pass's tokens (a few KiB-long rows per wave),
            // then its weights.  Loads retire in issue order, so chunk c
            // waits for what was issued up to its own weights and no token
            // load's latency is left exposed between chunks.
            u32x4 xs[TOK_PASS][XPW], wv[TOK_PASS][RPW];
#pragma unroll
            for (int c = 0; c < TOK_PASS; ++c) load_x(c, xs[c]);
            __builtin_amdgcn_sched_barrier(0);
            load_w(wv);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int c = 0; c < TOK_PASS; ++c) chunk(c, wv[c], xs[c]);
        } else if (full) {
            // Issue order: the token fragments of chunks 0 and 1, the pass's
            // weights, then the fragments of chunk c + 2 once chunk c's MFMAs
            // have read that register set: chunk 0 waits for its weights, not
            // for the whole pass.
            u32x4 xa[XPW], xb[XPW], wv[TOK_PASS][RPW];
            load_x(0, xa);
            load_x(1, xb);
            __builtin_amdgcn_sched_barrier(0);
            load_w(wv);
            __builtin_amdgcn_sched_barrier(0);
            chunk(0, wv[0], xa);
            __builtin_amdgcn_sched_barrier(0);
            load_x(2, xa);
            chunk(1, wv[1], xb);
            __builtin_amdgcn_sched_barrier(0);
            load_x(3, xb);
            chunk(2, wv[2], xa);
            chunk(3, wv[3], xb);
        } else {
            u32x4 xr[XPW];
            // the last pass (or any, past the buffer path's offsets): bounded
            // loads chunk by chunk (chunks past K skipped)
            for (int c = 0; c < TOK_PASS && p0 + c * TOK_KC < K; ++c) {
                u32x4 w[RPW];
#pragma unroll
                for (int j = 0; j < RPW; ++j)
                    w[j] = load16_row<false>(wrow[j] + p0 + c * TOK_KC + 16 * lane, wrow[j] + K);
                load_x(c, xr);
                chunk(c, w, xr);
            }
        }
    }

    // sum the four waves' partial products (exact INT32) through the chunk
    // buffer, once every wave is done reading it
    __syncthreads();
    int* const partial = reinterpret_cast<int*>(wt);     // [3][16][64]
    if (wave > 0) {
#pragma unroll
        for (int r = 0; r < 16; ++r) partial[((wave - 1) * 16 + r) * 64 + lane] = acc[r];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int w = 0; w < TOK_WAVES - 1; ++w)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] += partial[(w * 16 + r) * 64 + lane];

    w8a8_epilogue(g, acc, o0 + r32, half);
}

// ---------------------------------------------------------------------------
// Up to 16 tokens over whole passes (K a multiple of 4096, X and W rows 16-byte
// aligned): the weights stream as in the one-token kernel, every load one
// contiguous KiB of one row, all of a wave's loads issued at once, row after
// row, non-temporal.  A workgroup of 14 wavefronts owns 56 channels, four
// weight rows (16 KiB per pass) per wave, so the 14336-channel layer is 256
// workgroups, one per CU, all resident from the start.  Measured against
// this shape: eight rows per wave in four-wave workgroups (the kernel above)
// streams the same bytes about a third slower, and two 28-channel workgroups
// per CU do not fit side by side at this register count, so half of them
// started only when the first half ended.
//
// The pass's token rows go straight to LDS first (direct loads, 16 rows x 4
// KiB), and each MFMA wave takes its K part of them into registers.  Then
// four phases: in phase j every wave writes its j-th weight row (4 KiB) to
// LDS, so the 14 rows staged are channels 4 w + j (w = 0..13) of the
// workgroup, the block of a 16x16x64 INT8 MFMA (16 tokens x 16 channels;
// operand rows 14 and 15 are dead rows whose sums are never written).  Eight
// waves take 512 K bytes each, eight steps of 64 bytes, into one register
// quad per phase.  The phases alternate between two LDS buffers (the second
// is the token buffer once the MFMA waves hold their tokens), so one barrier
// per phase suffices, and a phase waits only for the weight row it stages,
// which each wave requested as one contiguous run before the next.  Every
// phase waits for the slowest wave's row, so phases start late in the
// stream; what a phase costs is then its LDS traffic, which holding the
// tokens in registers halves.  The eight K parts of each block meet in LDS
// at the end.
// ---------------------------------------------------------------------------
constexpr int TS_WAVES = 14;                                  // wavefronts per workgroup
constexpr int TS_RPW = 4;                                     // weight rows per wave (= phases)
constexpr int TS_CH = TS_RPW * TS_WAVES;                      // live channels per workgroup (56)
constexpr int TS_PITCH = TOK_PASS * TOK_KC + 16;              // LDS row pitch: a pass + 16 bytes
constexpr int TS_XP = (16 + TS_WAVES - 1) / TS_WAVES;         // token rows per wave (direct loads)
constexpr int TS_MW = 8;                                      // MFMA waves: 8 K parts of 512 bytes

__global__ __launch_bounds__(64 * TS_WAVES) void gemm_w8a8_stream_kernel(W8A8Args g) {
    // two buffers of 16 rows of a pass: st[0] holds the weight rows of even
    // phases, st[1] the token rows and then the weight rows of odd phases
    __shared__ __attribute__((aligned(16))) char st[2][16 * TS_PITCH];
    // the epilogue's weight scales, bias and token scales per phase block
    __shared__ float esc[TS_RPW][3][64];
    static_assert(TS_MW * TS_RPW * 4 * 64 * 4 <= 16 * TS_PITCH, "partial sums fit");
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int o0 = blockIdx.x * TS_CH;
    MPDT_LDS char* const sl = lds_cast(&st[0][0]);
    MPDT_LDS char* const xl = sl + 16 * TS_PITCH;   // the token rows (buffer 1)

    // Buffer resources with scalar bases and offsets and one lane offset for
    // every load (the host checks that the offset sums stay below 2^32).
    // This wave's weight rows: rows 4 w .. 4 w + 3 of the workgroup's (a row
    // past N reads row N - 1; its channel is never written).
    const int wr0 = min(o0 + TS_RPW * wave, g.N - 1);
    uint32_t wro[TS_RPW];
#pragma unroll
    for (int j = 0; j < TS_RPW; ++j)
        wro[j] = (uint32_t)((int64_t)(min(o0 + TS_RPW * wave + j, g.N - 1) - wr0) * g.ldw);
    const __amdgpu_buffer_rsrc_t wrs = buffer_rsrc((const char*)g.W + (int64_t)wr0 * g.ldw, 0xffffffffu);
    const i32x4 xrs = rsrc_words((uint64_t)(uintptr_t)g.X, 0xffffffffu);
    const uint32_t lane16 = 16u * (uint32_t)lane;
    const uint32_t ldx = (uint32_t)g.ldx;
    // MFMA operands: token row / staged row lane % 16, 16 K bytes at
    // 16 (lane / 16) of each 64-byte step of this wave's K part
    const uint32_t lo = (uint32_t)((lane & 15) * TS_PITCH + 512 * (wave & (TS_MW - 1)) + 16 * (lane >> 4));

    // The epilogue's scales and bias, fetched straight into LDS before any
    // other load (fetched at the end, they would add a memory round trip
    // after the last weights arrive), by the wave that writes block j: lane l
    // takes channel 4 (l % 16) + j of the workgroup and token l % 16.
    // Channels past N and tokens past M fall outside the buffers' ranges and
    // read zero without touching memory.
    if (wave < TS_RPW) {
        const int j = wave;
        const uint32_t nch = (uint32_t)min((int64_t)(g.N - o0) * 4, (int64_t)0xffffffff);
        const uint32_t lc = 4u * (uint32_t)(TS_RPW * (lane & 15) + j);
        const uint32_t l4 = 4u * (uint32_t)(lane & 15);
        lds_dma4(rsrc_words((uint64_t)(uintptr_t)(g.w_scale + o0), nch), lds_cast(&esc[j][0][0]), lc, 0u);
        if (g.bias) lds_dma4(rsrc_words((uint64_t)(uintptr_t)(g.bias + o0), nch), lds_cast(&esc[j][1][0]), lc, 0u);
        lds_dma4(rsrc_words((uint64_t)(uintptr_t)g.x_scale, 4u * (uint32_t)g.M), lds_cast(&esc[j][2][0]), l4, 0u);
    }

    i32x4 acc[TS_RPW];
#pragma unroll
    for (int j = 0; j < TS_RPW; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[j][r] = 0;
    for (int64_t p0 = 0; p0 < g.K; p0 += (int64_t)TOK_PASS * TOK_KC) {
        const uint32_t pk = (uint32_t)p0;
        if (p0 > 0) __syncthreads();           // the previous pass's reads are done
        // The pass's token rows straight into LDS (no registers held): wave w
        // loads rows w and w + 14 (below M), four KiB each.  Issued before the
        // weights, so they have landed once a wave has waited for all but its
        // weight loads (loads retire in issue order).
#pragma unroll
        for (int i = 0; i < TS_XP; ++i) {
            const int m = wave + TS_WAVES * i;
            if (m < 16 && m < g.M) {
#pragma unroll
                for (int c = 0; c < TOK_PASS; ++c)
                    lds_dma16(xrs, xl + m * TS_PITCH + c * TOK_KC, lane16,
                              (uint32_t)m * ldx + pk + (uint32_t)(c * TOK_KC));
            }
        }
        // the weights, row after row (each row one contiguous run of four
        // KiB), non-temporal (aux 2)
        u32x4 wv[TS_RPW][TOK_PASS];
#pragma unroll
        for (int j = 0; j < TS_RPW; ++j) {
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int c = 0; c < TOK_PASS; ++c)
                wv[j][c] = __builtin_bit_cast(
                    u32x4, __builtin_amdgcn_raw_buffer_load_b128(wrs, lane16, wro[j] + pk + c * TOK_KC, 2));
        }
        __builtin_amdgcn_sched_barrier(0);
        wait_vmem<TS_RPW * TOK_PASS>();            // this wave's token rows have landed
        __syncthreads();                           // everyone's
        // this MFMA wave's tokens for the pass: its K part, eight steps
        u32x4 xa[8];
        if (wave < TS_MW) {
#pragma unroll
            for (int s = 0; s < 8; ++s) xa[s] = lds_load16(xl, lo + 64 * s);
        }
#pragma unroll
        for (int j = 0; j < TS_RPW; ++j) {
            // phase j stages in buffer j % 2; the waves' reads of that buffer
            // (the tokens, or phase j - 2) ended before the previous barrier
            MPDT_LDS char* const wl = sl + (j & 1) * 16 * TS_PITCH;
#pragma unroll
            for (int c = 0; c < TOK_PASS; ++c)
                lds_store16(wl, (uint32_t)(wave * TS_PITCH + c * TOK_KC) + lane16, wv[j][c]);
            __syncthreads();
            if (wave < TS_MW) {
                // weight operands read two steps ahead of their MFMA
                u32x4 b0 = lds_load16(wl, lo), b1 = lds_load16(wl, lo + 64);
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    u32x4 b2 = b1;
                    if (s + 2 < 8) b2 = lds_load16(wl, lo + 64 * (s + 2));
                    acc[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, xa[s]),
                                                                   __builtin_bit_cast(i32x4, b0), acc[j], 0, 0, 0);
                    b0 = b1;
                    b1 = b2;
                }
            }
        }
    }

    // the eight K parts of each block (exact INT32) through the even-phase
    // buffer, once every wave is done reading it; wave j adds block j's and
    // writes its 14 channels
    __syncthreads();
    int* const partial = reinterpret_cast<int*>(&st[0][0]);   // [8 K parts][4 blocks][4][64]
    if (wave < TS_MW) {
#pragma unroll
        for (int j = 0; j < TS_RPW; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) partial[((wave * TS_RPW + j) * 4 + r) * 64 + lane] = acc[j][r];
    }
    __syncthreads();
    if (wave >= TS_RPW) return;
    const int j = wave;
    i32x4 z4 = {0, 0, 0, 0};
#pragma unroll
    for (int w = 0; w < TS_MW; ++w)
#pragma unroll
        for (int r = 0; r < 4; ++r) z4[r] += partial[((w * TS_RPW + j) * 4 + r) * 64 + lane];
    const int row = lane & 15;                 // staged row: channel 4 row + j of the workgroup
    const int o = o0 + TS_RPW * row + j;
    if (row >= TS_WAVES || o >= g.N) return;   // dead operand rows, channels past N
    const float sw = esc[j][0][row];
    const float bo = esc[j][1][row];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int m = 4 * (lane >> 4) + r;    // sum r of lane l: token 4 (l / 16) + r
        if (m < g.M) {
            const int z = z4[r];
            if (g.Z) g.Z[(int64_t)m * g.ldz + o] = z;
            // three separately rounded FP32 operations (no fused multiply-add)
            float v = mul_rn((float)z, esc[j][2][m]);
            v = mul_rn(v, sw);
            if (g.bias) v = add_rn(v, bo);
            if (g.Q) {
                // requantised: one IEEE division, round half to even, saturate to +-127
                const float q = __builtin_rintf(v / g.q_scale);
                g.Q[(int64_t)m * g.ldq + o] = (int8_t)fminf(fmaxf(q, -127.0f), 127.0f);
            } else {
                g.Y[(int64_t)m * g.ldy + o] = f32_to_bf16_bits(v);
            }
        }
    }
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

hipError_t launch_gemm_w8a8(const W8A8Args& a0, bool aligned, hipStream_t stream) {
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
            dim3 grid((unsigned)((a.N + TOK_CH - 1) / TOK_CH)), block(64 * TOK_WAVES);
            // (the streaming kernel adds 32-bit buffer offsets: row offsets plus K)
            const bool fits32 = (int64_t)(a.M - 1) * a.ldx + a.K + 4096 < (int64_t(1) << 32) &&
                                (int64_t)(TS_RPW - 1) * a.ldw + a.K + 4096 < (int64_t(1) << 32);
            if (a.M <= 16 && aligned && fits32 && a.K > 0 && a.K % (TOK_PASS * TOK_KC) == 0)
                hipLaunchKernelGGL(gemm_w8a8_stream_kernel, dim3((unsigned)((a.N + TS_CH - 1) / TS_CH)),
                                   dim3(64 * TS_WAVES), 0, stream, a);
            else if (a.M <= 16) hipLaunchKernelGGL(gemm_w8a8_kernel<true>, grid, block, 0, stream, a);
            else hipLaunchKernelGGL(gemm_w8a8_kernel<false>, grid, block, 0, stream, a);
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace mpdt
