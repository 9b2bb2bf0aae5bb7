// probes.hip -- libmpdt_probes.so: single-wavefront kernels that pin the
// gfx950 lane layouts the GEMM kernels rely on.  Used only by the test-suite;
// every probe touches a fixed, small, in-bounds set of addresses.
//
//   mpdt_probe_tr(bits, lds_image, offsets, out): copies a 4 KiB image into
//     LDS, then each of the 64 lanes issues one transposing read
//     (ds_read_b64_tr_b16 when bits == 16, ds_read_b64_tr_b8 when bits == 8)
//     at its byte offset and writes the 8 bytes it received to out[lane].
//   mpdt_probe_mfma(kind, A, B, D): one MFMA of the GEMM kernels (kind 0 f16
//     32x32x16, 1 bf16 32x32x16, 2 i8 32x32x32, 3 fp8 e4m3 32x32x64) with A
//     (32 x KS, row-major) and B (KS x 32, row-major) loaded with the lane
//     mapping the GEMM kernels use (lane l: row / column l % 32, K elements
//     [KS/2 * (l/32), KS/2 * (l/32 + 1)) in order), D (32 x 32, row-major,
//     FP32 or INT32) stored with the accumulator mapping the GEMM epilogue
//     uses (register r of lane l is row 8*(r/4) + 4*(l/32) + r%4, column l%32).
//   mpdt_probe_unaligned(src, off, soff, range, out_dma, out_ld): lane l moves
//     bytes [soff + off + 16 l, +16) of src once with a direct-to-LDS buffer
//     load (lane offset off + 16 l, scalar offset soff; then LDS ->
//     out_dma[l]) and once with a plain 16-byte load (-> out_ld[l]); neither
//     offset need be a multiple of 16.  With range < soff + off + 1024 it also
//     shows which offsets the buffer range check covers.
//   mpdt_probe_stream_read(p, bytes, per_lane, waves, out): the practical
//     HBM read ceiling -- every 16-byte chunk of [p, p + bytes) is read once
//     with non-temporal 16-byte loads, a wave taking per_lane KiB in a row
//     (lane l reads chunks l, l + 64, ... of its KiB runs, all loads issued
//     before any is used; bytes must hold at least one wave's per_lane KiB),
//     `waves` wavefronts per workgroup; only a value no
//     real sum takes is ever written, so the kernel moves almost nothing but
//     the reads.  Not a probe of layout: a measuring stick for the streaming
//     kernels (the W8A8 GEMV reads its weights this way, 8 KiB per wave).
//   mpdt_probe_mfma_peak(kind, data, iters, out, stamps): the practical MFMA
//     ceiling -- 256 workgroups of four wavefronts (one per SIMD, as the
//     one-wave GEMM kernels run), each wavefront 16 independent 32 x 32
//     accumulators and eight register-held pairs of operand fragments taken
//     from `data`, then iters x 128 back-to-back MFMAs of one kind (BF16
//     32x32x16, FP8 E4M3 32x32x64 with unit scales, INT8 32x32x32) whose B
//     operand changes at every instruction, and nothing else.  BF16 at iters
//     = 32: a wavefront issues the 4096 MFMAs of the BF16 4096^3 GEMM.  out[workgroup * 256 + thread] = the sum of the
//     thread's accumulators (keeps every MFMA); stamps[workgroup * 4 ..] =
//     s_memtime and s_memrealtime (100 MHz) at the start and the end of
//     workgroup's first wavefront, for the shader clock under this load.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <type_traits>

#include "device_common.hpp"

#define MPDT_EXPORT extern "C" __attribute__((visibility("default")))

namespace mpdt {

__global__ __launch_bounds__(64) void probe_tr_kernel(int bits, const u32x4* image,
                                                      const uint32_t* offsets, u32x2* out) {
    __shared__ __attribute__((aligned(16))) char smem[4096];
    MPDT_LDS char* lds = lds_cast(smem);
    const int lane = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 4; ++i) lds_store16(lds, 16 * (lane + 64 * i), image[lane + 64 * i]);
    __syncthreads();
    const uint32_t off = offsets[lane] & (4096u - 8u);
    out[lane] = (bits == 16) ? lds_read_tr16(lds, off) : lds_read_tr8(lds, off);
}

__global__ __launch_bounds__(64) void probe_unaligned_kernel(const char* src, uint32_t off, uint32_t soff,
                                                             uint32_t range, u32x4* out_dma, u32x4* out_ld) {
    __shared__ __attribute__((aligned(1024))) char smem[1024];
    MPDT_LDS char* lds = lds_cast(smem);
    const int lane = threadIdx.x;
    const i32x4 r = rsrc_words((uint64_t)(uintptr_t)src, range);
    lds_dma16<0, true>(r, lds, off + 16u * (uint32_t)lane, soff);
    __builtin_amdgcn_s_waitcnt(0);   // every counter at zero: the direct load has landed
    __syncthreads();
    out_dma[lane] = lds_load16(lds, 16u * (uint32_t)lane);
    out_ld[lane] = *reinterpret_cast<const u32x4*>(src + soff + off + 16u * (uint32_t)lane);
}

template <int KIND>
__global__ __launch_bounds__(64) void probe_mfma_kernel(const char* A, const char* B, void* D) {
    const int l = threadIdx.x;
    const int row = l & 31, half = l >> 5;
    if constexpr (KIND <= 2) {
        // 16 bytes of K per lane: f16/bf16 8 elements, i8 16 elements
        constexpr int ES = (KIND <= 1) ? 2 : 1;
        constexpr int KS = 32 / ES;                 // K of the instruction
        u32x4 a, b;
        for (int w = 0; w < 4; ++w) {
            uint32_t av = 0, bv = 0;
            for (int q = 0; q < 4 / ES; ++q) {
                const int k = half * (KS / 2) + w * (4 / ES) + q;
                uint32_t ea = 0, eb = 0;
                if (ES == 2) {
                    ea = ((const uint16_t*)A)[row * KS + k];
                    eb = ((const uint16_t*)B)[k * 32 + row];
                } else {
                    ea = ((const uint8_t*)A)[row * KS + k];
                    eb = ((const uint8_t*)B)[k * 32 + row];
                }
                av |= ea << (8 * ES * q);
                bv |= eb << (8 * ES * q);
            }
            a[w] = av;
            b[w] = bv;
        }
        if constexpr (KIND == 0) {
            f32x16 c = {};
            c = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                       __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
            for (int r = 0; r < 16; ++r)
                ((float*)D)[(8 * (r >> 2) + 4 * half + (r & 3)) * 32 + row] = c[r];
        } else if constexpr (KIND == 1) {
            f32x16 c = {};
            c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                        __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
            for (int r = 0; r < 16; ++r)
                ((float*)D)[(8 * (r >> 2) + 4 * half + (r & 3)) * 32 + row] = c[r];
        } else {
            i32x16 c = {};
            c = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, a),
                                                      __builtin_bit_cast(i32x4, b), c, 0, 0, 0);
            for (int r = 0; r < 16; ++r)
                ((int32_t*)D)[(8 * (r >> 2) + 4 * half + (r & 3)) * 32 + row] = c[r];
        }
    } else {
        // FP8: 32 bytes of K per lane, K = 64
        i32x8 a, b;
        for (int w = 0; w < 8; ++w) {
            uint32_t av = 0, bv = 0;
            for (int q = 0; q < 4; ++q) {
                const int k = half * 32 + w * 4 + q;
                av |= (uint32_t)((const uint8_t*)A)[row * 64 + k] << (8 * q);
                bv |= (uint32_t)((const uint8_t*)B)[k * 32 + row] << (8 * q);
            }
            a[w] = (int32_t)av;
            b[w] = (int32_t)bv;
        }
        f32x16 c = {};
        // kind 3: E4M3 x E4M3; kind 4: E5M2 x E5M2 (the instruction's format fields)
        if constexpr (KIND == 3) c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
        else c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 1, 1, 0, 127, 0, 127);
        for (int r = 0; r < 16; ++r)
            ((float*)D)[(8 * (r >> 2) + 4 * half + (r & 3)) * 32 + row] = c[r];
    }
}

// The wave's window of PER * 64 chunks is moved back to end at the buffer's
// last chunk when it would pass it (the host launches only buffers of at
// least one window), so no load leaves the buffer whatever the grid and the
// loads carry no branches: a conditional load lets the compiler place a wait
// between two loads, which leaves most of a wave's bytes unrequested until
// the first ones arrive.  Chunks that the moved window shares with the wave
// before it are left out of the sum.
template <int PER>
__global__ __launch_bounds__(1024) void probe_stream_read_kernel(const u32x4* p, uint64_t n16, uint32_t* out) {
    const uint64_t wave = (uint64_t)blockIdx.x * (blockDim.x >> 6) +
                          (uint64_t)__builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint64_t lane = threadIdx.x & 63;
    constexpr uint64_t SPAN = (uint64_t)PER * 64;
    const uint64_t first = wave * SPAN;
    const uint64_t base = first + SPAN <= n16 ? first : n16 - SPAN;
    const u32x4* q = p + base + lane;
    u32x4 v[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) v[i] = __builtin_nontemporal_load(q + 64 * i);
    // every load of the wave is issued before the first wait
    __builtin_amdgcn_sched_barrier(0);
    uint32_t acc = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i)
        if (base + (uint64_t)i * 64 + lane >= first) acc ^= v[i][0] ^ v[i][1] ^ v[i][2] ^ v[i][3];
    if (acc == 0x9E3779B9u && lane == 0) out[0] = acc;   // keeps the loads; (practically) never stores
}

constexpr int PEAK_WGS = 256;

// KIND 0: 32x32x16 BF16 (operands 16 bytes a lane); 1: 32x32x64 FP8 E4M3
// with unit block scales (32 bytes); 2: 32x32x32 INT8 (16 bytes).
template <int KIND>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void probe_mfma_peak_kernel(const u32x4* data, int iters, float* out, uint64_t* stamps) {
    constexpr int V = KIND == 1 ? 2 : 1;         // 16-byte pieces per operand fragment
    using Acc = typename std::conditional<KIND == 2, i32x16, f32x16>::type;
    const int lane = threadIdx.x & 63;
    u32x4 a[8][V], b[8][V];
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
        for (int v = 0; v < V; ++v) {
            a[s][v] = data[(s * V + v) * 64 + lane];
            b[s][v] = data[512 + (s * V + v) * 64 + lane];
        }
    Acc acc[16];
#pragma unroll
    for (int k = 0; k < 16; ++k)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[k][r] = 0;
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_sched_barrier(0);
    const uint64_t t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    __builtin_amdgcn_sched_barrier(0);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int s = 0; s < 8; ++s)
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const int t = (s + k) & 7;
                if constexpr (KIND == 0) {
                    acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[s][0]),
                                                                     __builtin_bit_cast(bf16x8, b[t][0]),
                                                                     acc[k], 0, 0, 0);
                } else if constexpr (KIND == 1) {
                    i32x8 a8, b8;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        a8[e] = (int32_t)a[s][e >> 2][e & 3];
                        b8[e] = (int32_t)b[t][e >> 2][e & 3];
                    }
                    acc[k] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, acc[k], 0, 0, 0, 127, 0, 127);
                } else {
                    acc[k] = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, a[s][0]),
                                                                   __builtin_bit_cast(i32x4, b[t][0]),
                                                                   acc[k], 0, 0, 0);
                }
            }
    }
    __builtin_amdgcn_sched_barrier(0);
    float sum = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k)
#pragma unroll
        for (int r = 0; r < 16; ++r) sum += (float)acc[k][r];
    const uint64_t t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
    out[blockIdx.x * 256 + threadIdx.x] = sum;
    if (threadIdx.x == 0) {
        uint64_t* q = stamps + blockIdx.x * 4;
        q[0] = t0; q[1] = t1; q[2] = r0; q[3] = r1;
    }
}

}  // namespace mpdt

// kind 0 BF16, 1 FP8 E4M3, 2 INT8; data: 2048 x 16 bytes of operand bits
// (BF16 and INT8 read the first 1024 and 512 + the next 512, FP8 all);
// out: 256 x 256 floats; stamps: 256 x 4 values.
MPDT_EXPORT int mpdt_probe_mfma_peak(int kind, const void* data, int iters, float* out, uint64_t* stamps,
                                     void* stream) {
    if (!data || !out || !stamps || iters < 0 || iters > (1 << 20)) return (int)hipErrorInvalidValue;
    const dim3 g(mpdt::PEAK_WGS), b(256);
    hipStream_t s = (hipStream_t)stream;
    const mpdt::u32x4* d = (const mpdt::u32x4*)data;
    switch (kind) {
        case 0: hipLaunchKernelGGL(mpdt::probe_mfma_peak_kernel<0>, g, b, 0, s, d, iters, out, stamps); break;
        case 1: hipLaunchKernelGGL(mpdt::probe_mfma_peak_kernel<1>, g, b, 0, s, d, iters, out, stamps); break;
        case 2: hipLaunchKernelGGL(mpdt::probe_mfma_peak_kernel<2>, g, b, 0, s, d, iters, out, stamps); break;
        default: return (int)hipErrorInvalidValue;
    }
    return (int)hipGetLastError();
}

MPDT_EXPORT int mpdt_probe_stream_read(const void* p, uint64_t bytes, int per_lane, int waves,
                                       uint32_t* out, void* stream) {
    if (waves < 1 || waves > 16 || !p || !out) return (int)hipErrorInvalidValue;
    const uint64_t n16 = bytes / 16;
    if (n16 == 0) return 0;
    const uint64_t per_wave = (uint64_t)per_lane * 64;
    if (n16 < per_wave) return (int)hipErrorInvalidValue;   // smaller than one wave's window
    const uint64_t nwaves = (n16 + per_wave - 1) / per_wave;
    const uint64_t grid = (nwaves + waves - 1) / waves;
    if (grid > 0x7fffffffull) return (int)hipErrorInvalidValue;
    const dim3 g((unsigned)grid), b((unsigned)(64 * waves));
    hipStream_t s = (hipStream_t)stream;
    const mpdt::u32x4* q = (const mpdt::u32x4*)p;
    switch (per_lane) {
        case 4: hipLaunchKernelGGL(mpdt::probe_stream_read_kernel<4>, g, b, 0, s, q, n16, out); break;
        case 8: hipLaunchKernelGGL(mpdt::probe_stream_read_kernel<8>, g, b, 0, s, q, n16, out); break;
        case 16: hipLaunchKernelGGL(mpdt::probe_stream_read_kernel<16>, g, b, 0, s, q, n16, out); break;
        default: return (int)hipErrorInvalidValue;
    }
    return (int)hipGetLastError();
}

MPDT_EXPORT int mpdt_probe_tr(int bits, const void* image, const uint32_t* offsets, void* out,
                              void* stream) {
    if (bits != 8 && bits != 16) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(mpdt::probe_tr_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, bits,
                       (const mpdt::u32x4*)image, offsets, (mpdt::u32x2*)out);
    return (int)hipGetLastError();
}

MPDT_EXPORT int mpdt_probe_mfma(int kind, const void* A, const void* B, void* D, void* stream) {
    const char* a = (const char*)A;
    const char* b = (const char*)B;
    hipStream_t s = (hipStream_t)stream;
    switch (kind) {
        case 0: hipLaunchKernelGGL(mpdt::probe_mfma_kernel<0>, dim3(1), dim3(64), 0, s, a, b, D); break;
        case 1: hipLaunchKernelGGL(mpdt::probe_mfma_kernel<1>, dim3(1), dim3(64), 0, s, a, b, D); break;
        case 2: hipLaunchKernelGGL(mpdt::probe_mfma_kernel<2>, dim3(1), dim3(64), 0, s, a, b, D); break;
        case 3: hipLaunchKernelGGL(mpdt::probe_mfma_kernel<3>, dim3(1), dim3(64), 0, s, a, b, D); break;
        case 4: hipLaunchKernelGGL(mpdt::probe_mfma_kernel<4>, dim3(1), dim3(64), 0, s, a, b, D); break;
        default: return (int)hipErrorInvalidValue;
    }
    return (int)hipGetLastError();
}

// size: bytes of src; every byte either load may touch lies inside it.
MPDT_EXPORT int mpdt_probe_unaligned(const void* src, uint32_t size, uint32_t off, uint32_t soff,
                                     uint32_t range, void* out_dma, void* out_ld, void* stream) {
    if ((uint64_t)soff + off + 1024u > size || range > size) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(mpdt::probe_unaligned_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream,
                       (const char*)src, off, soff, range, (mpdt::u32x4*)out_dma, (mpdt::u32x4*)out_ld);
    return (int)hipGetLastError();
}
