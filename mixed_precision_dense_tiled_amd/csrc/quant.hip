// quant.hip -- the quantisation steps on either side of the low-precision
// matrix paths, for gfx950:
//
//   * per-token symmetric INT8 quantisation of BF16 activations, the step that
//     produces q_x and s_x for the W8A8 layer ("NVIDIA A100: from chip to
//     SIMT", section 5.1: symmetric, zero point 0, one scale per token, made
//     at run time by the previous operator or a separate quantisation step):
//       s = amax_k |x[m][k]| / 127   (1 for an all-zero row)
//       q[m][k] = clamp(rne(x[m][k] / s), -127, 127)
//   * FP8 quantisation, the scale factors FP8 needs ("Tensor Core" page,
//     section "Precision": per tensor, per row or per block), in 1 x 128 or
//     128 x 128 blocks, or one scale per row, per column or per tensor, into
//     E4M3 (largest value 448) or E5M2 (57344):
//       s = amax_block |x| / qmax    (1 for an all-zero block)
//       q = fp8_rne(x / s)           (|x / s| <= qmax up to one rounding)
//
// Both are memory-bound elementwise passes with one reduction per row or
// block; every division is the IEEE-rounded FP32 one and rounding to an
// integer is v_rndne (ties to even).  The FP32 -> FP8 step is the gfx950
// conversion instruction (OCP E4M3 / E5M2, round to nearest even).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "device_common.hpp"
#include "kernels.hpp"

namespace mpdt {

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
    return v;
}

// maximum over the 256 threads of a workgroup (every thread gets it)
__device__ __forceinline__ float block_max256(float v, float* red) {
    v = wave_max(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = v;
    __syncthreads();
    const float r = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    return r;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __uint_as_float((uint32_t)b << 16);
}

// ---- per-token INT8 quantisation: one workgroup per token ------------------
// With vec rows up to I8_VK elements long, each thread loads its 16-byte
// pieces of the row once (all loads in flight together), keeps them in
// registers for the second pass and stores eight codes at once; otherwise
// the row is read twice, element by element.
constexpr int I8_VU = 4;                       // 16-byte pieces per thread
constexpr int64_t I8_VK = 256 * 8 * I8_VU;     // 8192 elements

__device__ __forceinline__ int8_t q_i8(float x, float s) {
    const float r = __builtin_rintf(x / s);
    return (int8_t)(int)fminf(fmaxf(r, -127.0f), 127.0f);
}

__global__ __launch_bounds__(256) void quantize_i8_rows_kernel(QuantI8Args g) {
    __shared__ float red[4];
    const int m = blockIdx.x;
    const uint16_t* xr = g.X + (int64_t)m * g.ldx;
    int8_t* qr = g.Q + (int64_t)m * g.ldq;
    if (g.vec && g.K <= I8_VK) {
        u32x4 v[I8_VU];
#pragma unroll
        for (int u = 0; u < I8_VU; ++u) {
            const int64_t k = 8 * (threadIdx.x + 256 * u);
            if (k + 8 <= g.K) {
                v[u] = *reinterpret_cast<const u32x4*>(xr + k);
            } else {
                v[u] = u32x4{0u, 0u, 0u, 0u};
                for (int e = 0; e < 8 && k + e < g.K; ++e) v[u][e >> 1] |= (uint32_t)xr[k + e] << (16 * (e & 1));
            }
        }
        float amax = 0.0f;
#pragma unroll
        for (int u = 0; u < I8_VU; ++u)
#pragma unroll
            for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(bf16_bits_to_f32((uint16_t)(v[u][e >> 1] >> (16 * (e & 1))))));
        amax = block_max256(amax, red);
        const float s = amax > 0.0f ? amax / 127.0f : 1.0f;
        if (threadIdx.x == 0) g.S[m] = s;
#pragma unroll
        for (int u = 0; u < I8_VU; ++u) {
            const int64_t k = 8 * (threadIdx.x + 256 * u);
            if (k >= g.K) break;
            uint32_t w[2] = {0u, 0u};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = bf16_bits_to_f32((uint16_t)(v[u][e >> 1] >> (16 * (e & 1))));
                w[e >> 2] |= (uint32_t)(uint8_t)q_i8(x, s) << (8 * (e & 3));
            }
            if (k + 8 <= g.K) {
                *reinterpret_cast<u32x2*>(qr + k) = u32x2{w[0], w[1]};
            } else {
                for (int e = 0; k + e < g.K; ++e) qr[k + e] = (int8_t)(w[e >> 2] >> (8 * (e & 3)));
            }
        }
        return;
    }
    float amax = 0.0f;
    for (int64_t k = threadIdx.x; k < g.K; k += 256) amax = fmaxf(amax, fabsf(bf16_bits_to_f32(xr[k])));
    amax = block_max256(amax, red);
    const float s = amax > 0.0f ? amax / 127.0f : 1.0f;
    if (threadIdx.x == 0) g.S[m] = s;
    for (int64_t k = threadIdx.x; k < g.K; k += 256) qr[k] = q_i8(bf16_bits_to_f32(xr[k]), s);
}

hipError_t launch_quantize_i8_rows(const QuantI8Args& a, hipStream_t stream) {
    if (a.M <= 0) return hipSuccess;
    hipLaunchKernelGGL(quantize_i8_rows_kernel, dim3((unsigned)a.M), dim3(256), 0, stream, a);
    return hipGetLastError();
}

// ---- FP8 block quantisation ----------------------------------------------
template <int FMT>
__device__ __forceinline__ uint8_t to_fp8(float v) {
    if constexpr (FMT == 0) return (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(v, 0.0f, 0, false) & 0xff);
    else return (uint8_t)(__builtin_amdgcn_cvt_pk_bf8_f32(v, 0.0f, 0, false) & 0xff);
}
template <int FMT> constexpr float QMAX = FMT == 0 ? 448.0f : 57344.0f;

// Four floats from c (a multiple of 4, 16-byte aligned in a vec row): one
// vector load inside [0, end), element loads (zeros past end) at the end.
__device__ __forceinline__ float4 load4_bounded(const float* xr, int64_t c, int64_t end) {
    if (c + 4 <= end) return *reinterpret_cast<const float4*>(xr + c);
    float4 v = {0.0f, 0.0f, 0.0f, 0.0f};
    if (c < end) v.x = xr[c];
    if (c + 1 < end) v.y = xr[c + 1];
    if (c + 2 < end) v.z = xr[c + 2];
    return v;
}
// 1 x 128 blocks: a wavefront takes FP8_RB = 4 consecutive blocks of one
// row.  With vec rows, lane l takes elements 4 l .. 4 l + 3 of each
// 256-element half (one 16-byte load; lanes 0-31 cover one block, 32-63
// the next), the maximum runs over each half-wave, and the four FP8 codes go
// out as one 4-byte store; otherwise two elements per lane and block, loaded
// and stored one at a time.  All loads are issued before the first
// reduction.
constexpr int FP8_RB = 4;

// four FP8 codes of v / s, element 0 in the low byte
template <int FMT>
__device__ __forceinline__ uint32_t fp8x4(float4 v, float s) {
    return (uint32_t)to_fp8<FMT>(v.x / s) | ((uint32_t)to_fp8<FMT>(v.y / s) << 8) |
           ((uint32_t)to_fp8<FMT>(v.z / s) << 16) | ((uint32_t)to_fp8<FMT>(v.w / s) << 24);
}

template <int FMT>
__global__ __launch_bounds__(256) void quantize_fp8_rowblocks_kernel(QuantFp8Args g) {
    const int64_t nbc = (g.C + 127) / 128;
    const int64_t groups = (nbc + FP8_RB - 1) / FP8_RB;              // block groups per row
    const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (w >= (int64_t)g.R * groups) return;         // whole wave: no barrier in this kernel
    const int lane = threadIdx.x & 63;
    const int64_t r = w / groups, bj0 = (w % groups) * FP8_RB;
    const float* xr = g.X + r * g.ldx;
    uint8_t* qr = g.Q + r * g.ldq;
    if (g.vec) {
        float4 v[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) v[h] = load4_bounded(xr, bj0 * 128 + 256 * h + 4 * lane, g.C);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int64_t bj = bj0 + 2 * h + (lane >> 5);   // this half-wave's block
            float amax = fmaxf(fmaxf(fabsf(v[h].x), fabsf(v[h].y)), fmaxf(fabsf(v[h].z), fabsf(v[h].w)));
#pragma unroll
            for (int m = 16; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
            if (bj >= nbc) continue;
            const float s = amax > 0.0f ? amax / QMAX<FMT> : 1.0f;
            if ((lane & 31) == 0) g.S[r * g.lds + bj] = s;
            const int64_t c = bj0 * 128 + 256 * h + 4 * lane;
            const uint32_t q = fp8x4<FMT>(v[h], s);
            if (c + 4 <= g.C) {
                *reinterpret_cast<uint32_t*>(qr + c) = q;
            } else {
                for (int e = 0; e < 4 && c + e < g.C; ++e) qr[c + e] = (uint8_t)(q >> (8 * e));
            }
        }
        return;
    }
    float v[FP8_RB][2];
#pragma unroll
    for (int b = 0; b < FP8_RB; ++b) {
        const int64_t c0 = (bj0 + b) * 128 + 2 * lane;
        v[b][0] = c0 < g.C ? xr[c0] : 0.0f;
        v[b][1] = c0 + 1 < g.C ? xr[c0 + 1] : 0.0f;
    }
#pragma unroll
    for (int b = 0; b < FP8_RB; ++b) {
        if (bj0 + b >= nbc) break;
        const int64_t c0 = (bj0 + b) * 128 + 2 * lane;
        const float amax = wave_max(fmaxf(fabsf(v[b][0]), fabsf(v[b][1])));
        const float s = amax > 0.0f ? amax / QMAX<FMT> : 1.0f;
        if (lane == 0) g.S[r * g.lds + bj0 + b] = s;
        if (c0 < g.C) qr[c0] = to_fp8<FMT>(v[b][0] / s);
        if (c0 + 1 < g.C) qr[c0 + 1] = to_fp8<FMT>(v[b][1] / s);
    }
}

// 128 x 128 blocks: one workgroup per block.  With vec rows thread t covers
// columns 4 (t % 32) .. +3 of the block's rows t / 32, t / 32 + 8, ... (one
// 16-byte load per row; a wave instruction reads 512 consecutive bytes of
// each of two rows) and stores four codes at once; otherwise column t % 128
// of rows t / 128, t / 128 + 2, ..., element by element.  The thread's 64
// values stay in registers between the two passes.
template <int FMT>
__global__ __launch_bounds__(256) void quantize_fp8_tileblocks_kernel(QuantFp8Args g) {
    __shared__ float red[4];
    const int64_t nbc = (g.C + 127) / 128;
    const int64_t bi = blockIdx.x / nbc, bj = blockIdx.x % nbc;
    if (g.vec) {
        const int64_t c = bj * 128 + 4 * (threadIdx.x & 31);
        const int64_t r0 = bi * 128 + (threadIdx.x >> 5);
        float4 v[16];
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int64_t r = r0 + 8 * i;
            v[i] = r < g.R ? load4_bounded(g.X + r * g.ldx, c, g.C) : float4{0.0f, 0.0f, 0.0f, 0.0f};
        }
#pragma unroll
        for (int i = 0; i < 16; ++i)
            amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)), fmaxf(fabsf(v[i].z), fabsf(v[i].w))));
        amax = block_max256(amax, red);
        const float s = amax > 0.0f ? amax / QMAX<FMT> : 1.0f;
        if (threadIdx.x == 0) g.S[bi * g.lds + bj] = s;
        if (c >= g.C) return;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int64_t r = r0 + 8 * i;
            if (r >= g.R) break;
            uint8_t* qr = g.Q + r * g.ldq;
            const uint32_t q = fp8x4<FMT>(v[i], s);
            if (c + 4 <= g.C) {
                *reinterpret_cast<uint32_t*>(qr + c) = q;
            } else {
                for (int e = 0; e < 4 && c + e < g.C; ++e) qr[c + e] = (uint8_t)(q >> (8 * e));
            }
        }
        return;
    }
    const int64_t c = bj * 128 + (threadIdx.x & 127);
    const int64_t r0 = bi * 128 + (threadIdx.x >> 7);
    const bool col_ok = c < g.C;
    float v[64];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 64; ++i) {
        const int64_t r = r0 + 2 * i;
        v[i] = (col_ok && r < g.R) ? g.X[r * g.ldx + c] : 0.0f;
        amax = fmaxf(amax, fabsf(v[i]));
    }
    amax = block_max256(amax, red);
    const float s = amax > 0.0f ? amax / QMAX<FMT> : 1.0f;
    if (threadIdx.x == 0) g.S[bi * g.lds + bj] = s;
    if (col_ok) {
#pragma unroll
        for (int i = 0; i < 64; ++i) {
            const int64_t r = r0 + 2 * i;
            if (r < g.R) g.Q[r * g.ldq + c] = to_fp8<FMT>(v[i] / s);
        }
    }
}

// One scale per row: a workgroup per row, the row read twice (maximum, then
// quantisation; the second pass mostly from cache).
template <int FMT>
__global__ __launch_bounds__(256) void quantize_fp8_perrow_kernel(QuantFp8Args g) {
    __shared__ float red[4];
    const int64_t r = blockIdx.x;
    const float* xr = g.X + r * g.ldx;
    uint8_t* qr = g.Q + r * g.ldq;
    float amax = 0.0f;
    for (int64_t c = threadIdx.x; c < g.C; c += 256) amax = fmaxf(amax, fabsf(xr[c]));
    amax = block_max256(amax, red);
    const float s = amax > 0.0f ? amax / QMAX<FMT> : 1.0f;
    if (threadIdx.x == 0) g.S[r * g.lds] = s;
    for (int64_t c = threadIdx.x; c < g.C; c += 256) qr[c] = to_fp8<FMT>(xr[c] / s);
}

// One scale per column: a workgroup per 64 columns, its four wavefronts on
// interleaved rows (each load instruction reads 256 consecutive bytes of a
// row), the four partial maxima of a column combined through LDS.
template <int FMT>
__global__ __launch_bounds__(256) void quantize_fp8_percol_kernel(QuantFp8Args g) {
    __shared__ float red[4][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t c = (int64_t)blockIdx.x * 64 + lane;
    const bool ok = c < g.C;
    float amax = 0.0f;
    if (ok)
        for (int64_t r = wave; r < g.R; r += 4) amax = fmaxf(amax, fabsf(g.X[r * g.ldx + c]));
    red[wave][lane] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0][lane], red[1][lane]), fmaxf(red[2][lane], red[3][lane]));
    const float s = amax > 0.0f ? amax / QMAX<FMT> : 1.0f;
    if (!ok) return;
    if (wave == 0) g.S[c] = s;
    for (int64_t r = wave; r < g.R; r += 4) g.Q[r * g.ldq + c] = to_fp8<FMT>(g.X[r * g.ldx + c] / s);
}

// One scale per tensor, in three launches on the stream: the maximum of every
// workgroup's part is folded into S[0] with an atomic maximum on its bit
// pattern (non-negative FP32 values order as unsigned integers), after S[0]
// was cleared; then every element is quantised with s = S[0] / qmax; then
// S[0] becomes s.
__global__ void fp8_tensor_clear_kernel(float* S) { S[0] = 0.0f; }

constexpr int TENSOR_WGS = 1024;   // workgroups of the two grid-stride passes

constexpr int TENSOR_CH = 4096;    // columns of one work item (a row piece)

// A work item is one row piece of TENSOR_CH columns; with aligned rows each
// thread reads four 16-byte vectors of it at once (16 KiB per workgroup in
// flight), else single elements.
__global__ __launch_bounds__(256) void fp8_tensor_amax_kernel(QuantFp8Args g) {
    __shared__ float red[4];
    float amax = 0.0f;
    const int64_t pieces = (g.C + TENSOR_CH - 1) / TENSOR_CH;
    for (int64_t it = blockIdx.x; it < g.R * pieces; it += gridDim.x) {
        const int64_t r = it / pieces, c0 = (it % pieces) * TENSOR_CH;
        const int64_t c1 = std::min<int64_t>(c0 + TENSOR_CH, g.C);
        const float* xr = g.X + r * g.ldx;
        if (g.vec) {
            float4 v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = load4_bounded(xr, c0 + 4 * (threadIdx.x + 256 * u), c1);
#pragma unroll
            for (int u = 0; u < 4; ++u)
                amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[u].x), fabsf(v[u].y)), fmaxf(fabsf(v[u].z), fabsf(v[u].w))));
        } else {
            for (int64_t c = c0 + threadIdx.x; c < c1; c += 256) amax = fmaxf(amax, fabsf(xr[c]));
        }
    }
    amax = block_max256(amax, red);
    if (threadIdx.x == 0) atomicMax((unsigned int*)g.S, __float_as_uint(amax));
}

template <int FMT>
__global__ __launch_bounds__(256) void fp8_tensor_quant_kernel(QuantFp8Args g) {
    const float amax = g.S[0];
    const float s = amax > 0.0f ? amax / QMAX<FMT> : 1.0f;
    const int64_t pieces = (g.C + TENSOR_CH - 1) / TENSOR_CH;
    for (int64_t it = blockIdx.x; it < g.R * pieces; it += gridDim.x) {
        const int64_t r = it / pieces, c0 = (it % pieces) * TENSOR_CH;
        const int64_t c1 = std::min<int64_t>(c0 + TENSOR_CH, g.C);
        const float* xr = g.X + r * g.ldx;
        uint8_t* qr = g.Q + r * g.ldq;
        if (g.vec) {
            float4 v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = load4_bounded(xr, c0 + 4 * (threadIdx.x + 256 * u), c1);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int64_t c = c0 + 4 * (threadIdx.x + 256 * u);
                const uint32_t q = (uint32_t)to_fp8<FMT>(v[u].x / s) | ((uint32_t)to_fp8<FMT>(v[u].y / s) << 8) |
                                   ((uint32_t)to_fp8<FMT>(v[u].z / s) << 16) | ((uint32_t)to_fp8<FMT>(v[u].w / s) << 24);
                if (c + 4 <= c1) {
                    *reinterpret_cast<uint32_t*>(qr + c) = q;
                } else {
                    for (int e = 0; e < 4 && c + e < c1; ++e) qr[c + e] = (uint8_t)(q >> (8 * e));
                }
            }
        } else {
            for (int64_t c = c0 + threadIdx.x; c < c1; c += 256) qr[c] = to_fp8<FMT>(xr[c] / s);
        }
    }
}

__global__ void fp8_tensor_scale_kernel(float* S, int fmt) {
    const float amax = S[0];
    S[0] = amax > 0.0f ? amax / (fmt == 0 ? QMAX<0> : QMAX<1>) : 1.0f;
}

template <int FMT>
static hipError_t launch_fp8q(const QuantFp8Args& a, hipStream_t stream) {
    const int64_t nbc = (a.C + 127) / 128;
    switch (a.shape) {
        case FP8Q_ROW128: {
            const int64_t waves = (int64_t)a.R * ((nbc + FP8_RB - 1) / FP8_RB);
            hipLaunchKernelGGL(quantize_fp8_rowblocks_kernel<FMT>, dim3((unsigned)((waves + 3) / 4)),
                               dim3(256), 0, stream, a);
            break;
        }
        case FP8Q_TILE128: {
            const int64_t nbr = (a.R + 127) / 128;
            hipLaunchKernelGGL(quantize_fp8_tileblocks_kernel<FMT>, dim3((unsigned)(nbr * nbc)), dim3(256),
                               0, stream, a);
            break;
        }
        case FP8Q_ROW:
            hipLaunchKernelGGL(quantize_fp8_perrow_kernel<FMT>, dim3((unsigned)a.R), dim3(256), 0, stream, a);
            break;
        case FP8Q_COL:
            hipLaunchKernelGGL(quantize_fp8_percol_kernel<FMT>, dim3((unsigned)((a.C + 63) / 64)), dim3(256),
                               0, stream, a);
            break;
        case FP8Q_TENSOR: {
            hipLaunchKernelGGL(fp8_tensor_clear_kernel, dim3(1), dim3(1), 0, stream, a.S);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            const int64_t wgs = std::min<int64_t>(TENSOR_WGS, a.R * ((a.C + TENSOR_CH - 1) / TENSOR_CH));
            hipLaunchKernelGGL(fp8_tensor_amax_kernel, dim3((unsigned)wgs), dim3(256), 0, stream, a);
            if ((e = hipGetLastError()) != hipSuccess) return e;
            hipLaunchKernelGGL(fp8_tensor_quant_kernel<FMT>, dim3((unsigned)wgs), dim3(256), 0, stream, a);
            if ((e = hipGetLastError()) != hipSuccess) return e;
            hipLaunchKernelGGL(fp8_tensor_scale_kernel, dim3(1), dim3(1), 0, stream, a.S, FMT);
            break;
        }
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_quantize_fp8_blocks(const QuantFp8Args& a, hipStream_t stream) {
    if (a.R <= 0 || a.C <= 0) return hipSuccess;
    return a.fmt == 0 ? launch_fp8q<0>(a, stream) : launch_fp8q<1>(a, stream);
}

}  // namespace mpdt
