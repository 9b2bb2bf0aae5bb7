// device_common.hpp -- small device-side building blocks shared by the GEMM
// and GEMV kernels: vector types, 16-byte row-segment loads with edge masking
// and re-alignment, and LDS address-space helpers.  gfx950 (CDNA4) only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mpdt {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(4))) int32_t i32x4;
typedef __attribute__((ext_vector_type(8))) int32_t i32x8;
typedef __attribute__((ext_vector_type(2))) int32_t i32x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) int32_t i32x16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) short i16x4;

#define MPDT_LDS __attribute__((address_space(3)))

__device__ __forceinline__ MPDT_LDS char* lds_cast(void* p) {
    return (MPDT_LDS char*)(p);
}

// Buffer resource (CDNA raw buffer, stride 0) over `range` bytes from a
// wave-uniform base: a buffer read at an offset at or past `range` returns
// zero and touches no memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t range) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)range,
                                             0x00020000 /* 32-bit data format (gfx9 family) */);
}

// 16 bytes per lane from buffer offset voff + soff straight into LDS: lane l's
// bytes land at dst + 16 * l (dst is wave-uniform).
__device__ __forceinline__ void buffer_to_lds16(__amdgpu_buffer_rsrc_t r, MPDT_LDS char* dst,
                                                uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (MPDT_LDS void*)dst, 16, (int)voff, (int)soff, 0, 0);
}

// Buffer resource words (raw buffer, stride 0, 32-bit data format) for
// `range` bytes from `base`; reads at offsets >= range return zero and touch
// no memory.
__device__ __forceinline__ i32x4 rsrc_words(uint64_t base, uint32_t range) {
    return i32x4{(int32_t)(uint32_t)base, (int32_t)((uint32_t)(base >> 32) & 0xffffu),
                 (int32_t)range, 0x00020000};
}

// 16 bytes per lane from buffer offset voff + soff + OFF into LDS at
// dst + OFF + 16 * lane (M0 = dst), written as inline assembly.  The compiler
// does not see this LDS write, so it adds no waits of its own before later LDS
// reads; the caller orders them with explicit vmcnt waits and workgroup
// barriers.  (The compiler's own tracking of direct-to-LDS loads falls back to
// waiting for every load in flight where control flow merges, which would
// empty a multi-stage pipeline at each loop entry.)  OFF (0..4095) moves both
// addresses, so several loads can share one M0 value.  NOP: the load may
// follow a write of M0 directly, which needs one wait state (s_nop 0) -- the
// first load after a new M0 value.
template <int OFF = 0, bool NOP = true>
__device__ __forceinline__ void lds_dma16(i32x4 r, MPDT_LDS char* dst, uint32_t voff,
                                          uint32_t soff) {
    static_assert(OFF >= 0 && OFF < 4096, "12-bit instruction offset");
    if constexpr (NOP)
        asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen offset:%4 lds"
                     :
                     : "{m0}"((uint32_t)(uintptr_t)dst), "v"(voff), "s"(r), "s"(soff), "n"(OFF));
    else
        asm volatile("buffer_load_dwordx4 %1, %2, %3 offen offset:%4 lds"
                     :
                     : "{m0}"((uint32_t)(uintptr_t)dst), "v"(voff), "s"(r), "s"(soff), "n"(OFF));
}

// 4-byte variant of lds_dma16: lane l's dword from buffer offset voff + soff +
// OFF lands at dst + OFF + 4 * l.  Same ordering rules.
template <int OFF = 0, bool NOP = true>
__device__ __forceinline__ void lds_dma4(i32x4 r, MPDT_LDS char* dst, uint32_t voff, uint32_t soff) {
    static_assert(OFF >= 0 && OFF < 4096, "12-bit instruction offset");
    if constexpr (NOP)
        asm volatile("s_nop 0\n\tbuffer_load_dword %1, %2, %3 offen offset:%4 lds"
                     :
                     : "{m0}"((uint32_t)(uintptr_t)dst), "v"(voff), "s"(r), "s"(soff), "n"(OFF));
    else
        asm volatile("buffer_load_dword %1, %2, %3 offen offset:%4 lds"
                     :
                     : "{m0}"((uint32_t)(uintptr_t)dst), "v"(voff), "s"(r), "s"(soff), "n"(OFF));
}

// s_waitcnt vmcnt(N): at most N vector-memory operations of this wave
// (direct-to-LDS loads included) are still in flight.  Memory reads retire in
// issue order, so this waits for all but the N most recent.
template <int N>
__device__ __forceinline__ void wait_vmem() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// s_waitcnt lgkmcnt(0): this wave's LDS reads and writes have completed.
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Keep the bytes [0, nbytes) of an 8-byte piece, zero the rest (nbytes 0..8).
__device__ __forceinline__ u32x2 mask_tail8(u32x2 v, int nbytes) {
#pragma unroll
    for (int w = 0; w < 2; ++w) {
        const int keep = nbytes - 4 * w;
        const uint32_t m = keep >= 4 ? 0xffffffffu : (keep <= 0 ? 0u : (0xffffffffu >> (8 * (4 - keep))));
        v[w] &= m;
    }
    return v;
}

// Zero the bytes [0, nbytes) of a 16-byte chunk / an 8-byte piece, keep the rest.
__device__ __forceinline__ u32x4 mask_head(u32x4 v, int nbytes) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const int drop = nbytes - 4 * w;   // bytes of dword w to clear
        const uint32_t m = drop >= 4 ? 0u : (drop <= 0 ? 0xffffffffu : (0xffffffffu << (8 * drop)));
        v[w] &= m;
    }
    return v;
}
__device__ __forceinline__ u32x2 mask_head8(u32x2 v, int nbytes) {
#pragma unroll
    for (int w = 0; w < 2; ++w) {
        const int drop = nbytes - 4 * w;
        const uint32_t m = drop >= 4 ? 0u : (drop <= 0 ? 0xffffffffu : (0xffffffffu << (8 * drop)));
        v[w] &= m;
    }
    return v;
}

// Keep the bytes [0, nbytes) of a 16-byte chunk, zero the rest (nbytes 0..16).
__device__ __forceinline__ u32x4 mask_tail(u32x4 v, int nbytes) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const int keep = nbytes - 4 * w;  // bytes of dword w to keep
        uint32_t m = keep >= 4 ? 0xffffffffu : (keep <= 0 ? 0u : (0xffffffffu >> (8 * (4 - keep))));
        v[w] &= m;
    }
    return v;
}

// 16 bytes starting at byte offset `off` (0..15) of the 32-byte pair (lo, hi).
__device__ __forceinline__ u32x4 extract16(u32x4 lo, u32x4 hi, int off) {
    const bool s2 = (off & 8) != 0, s1 = (off & 4) != 0;
    const uint32_t b = (uint32_t)(off & 3);
    // shift by two dwords, then by one, then by bytes
    const uint32_t e0 = s2 ? lo[2] : lo[0], e1 = s2 ? lo[3] : lo[1];
    const uint32_t e2 = s2 ? hi[0] : lo[2], e3 = s2 ? hi[1] : lo[3];
    const uint32_t e4 = s2 ? hi[2] : hi[0], e5 = s2 ? hi[3] : hi[1];
    const uint32_t f0 = s1 ? e1 : e0, f1 = s1 ? e2 : e1, f2 = s1 ? e3 : e2;
    const uint32_t f3 = s1 ? e4 : e3, f4 = s1 ? e5 : e4;
    u32x4 r;
    r[0] = __builtin_amdgcn_alignbyte(f1, f0, b);
    r[1] = __builtin_amdgcn_alignbyte(f2, f1, b);
    r[2] = __builtin_amdgcn_alignbyte(f3, f2, b);
    r[3] = __builtin_amdgcn_alignbyte(f4, f3, b);
    return r;
}

// Load the 16 bytes [p, p + 16) of a row whose valid bytes end at `end`
// (bytes at or past `end` read as zero).  ALIGNED: p is 16-byte aligned.
// Otherwise only aligned 16-byte chunks that contain at least one valid byte
// are read: such a chunk never leaves the memory page of that valid byte, so
// no access can fault, and the wanted bytes are shifted into place.
template <bool ALIGNED>
__device__ __forceinline__ u32x4 load16_row(const char* p, const char* end) {
    const long avail = end - p;
    if (avail <= 0) return u32x4{0u, 0u, 0u, 0u};
    if constexpr (ALIGNED) {
        u32x4 v = *reinterpret_cast<const u32x4*>(p);
        return avail >= 16 ? v : mask_tail(v, (int)avail);
    } else {
        const uintptr_t a = reinterpret_cast<uintptr_t>(p);
        const int off = (int)(a & 15u);
        const char* base = p - off;
        u32x4 lo = *reinterpret_cast<const u32x4*>(base);
        u32x4 hi = u32x4{0u, 0u, 0u, 0u};
        if (off != 0 && avail > 16 - off) hi = *reinterpret_cast<const u32x4*>(base + 16);
        u32x4 v = off ? extract16(lo, hi, off) : lo;
        return avail >= 16 ? v : mask_tail(v, (int)avail);
    }
}

// Unguarded aligned 16-byte load (interior of a tile).
__device__ __forceinline__ u32x4 load16_fast(const char* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ void lds_store16(MPDT_LDS char* base, uint32_t byte_off, u32x4 v) {
    *reinterpret_cast<MPDT_LDS u32x4*>(base + byte_off) = v;
}

__device__ __forceinline__ u32x4 lds_load16(const MPDT_LDS char* base, uint32_t byte_off) {
    return *reinterpret_cast<const MPDT_LDS u32x4*>(base + byte_off);
}

// Transposing LDS reads (gfx950).  Within each group of 16 lanes, every lane
// names one 8-byte piece of a small row-major block; lane q of the group
// receives column q of that block:
//   tr16: block of 4 rows x 16 16-bit elements, lane p names row p/4,
//         elements 4*(p%4)..+3; lane q gets rows 0..3 of column q.
//   tr8:  block of 8 rows x 16 bytes, lane p names row p/2, bytes
//         8*(p%2)..+7; lane q gets rows 0..7 of column q.
__device__ __forceinline__ u32x2 lds_read_tr16(const MPDT_LDS char* base, uint32_t byte_off) {
    auto p = (MPDT_LDS i16x4*)(base + byte_off);
    i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p);
    return __builtin_bit_cast(u32x2, r);
}

__device__ __forceinline__ u32x2 lds_read_tr8(const MPDT_LDS char* base, uint32_t byte_off) {
    auto p = (MPDT_LDS i32x2*)(base + byte_off);
    i32x2 r = __builtin_amdgcn_ds_read_tr8_b64_v2i32(p);
    return __builtin_bit_cast(u32x2, r);
}

// FP32 multiply and add, each rounded on its own: never contracted into a
// fused multiply-add with a neighbouring operation.
__device__ __forceinline__ float mul_rn(float a, float b) {
#pragma clang fp contract(off)
    return a * b;
}
__device__ __forceinline__ float add_rn(float a, float b) {
#pragma clang fp contract(off)
    return a + b;
}

// Round FP32 to FP16 (nearest, ties to even, subnormals kept, overflow to
// infinity) with the hardware conversion.
__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
    _Float16 h = (_Float16)x;
    return __builtin_bit_cast(uint16_t, h);
}

// Round FP32 to BF16 (nearest, ties to even) with the hardware conversion.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
    __bf16 h = (__bf16)x;
    return __builtin_bit_cast(uint16_t, h);
}

}  // namespace mpdt
