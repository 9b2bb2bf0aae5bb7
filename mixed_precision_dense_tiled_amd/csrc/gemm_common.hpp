// gemm_common.hpp -- pieces shared by the GEMM kernels (gemm_kernel.hpp,
// gemm_fp8.hip): MFMA traits, tile geometry, LDS swizzles, the workgroup
// to tile mapping and the wait / barrier primitives.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"

namespace mpdt {
#ifdef MPDT_CLOCK_STAMPS
// Instrumented build (a separate measurement library, never the product
// one): workgroup w < CLOCK_STAMP_WGS records the shader clock (s_memtime)
// and the 100 MHz real-time counter (s_memrealtime) at kernel entry, after
// the K loop and after its last store has completed -- enough to read the
// shader clock the kernel actually ran at and where its time went.
constexpr int CLOCK_STAMP_WGS = 4096;
// (one copy per translation unit: each exports its own reader)
static __device__ uint64_t g_clock_stamps[CLOCK_STAMP_WGS * 6];
#define MPDT_STAMP(i)                                        \
    const uint64_t stamp_t##i = __builtin_amdgcn_s_memtime(); \
    const uint64_t stamp_r##i = __builtin_amdgcn_s_memrealtime();
#else
#define MPDT_STAMP(i)
#endif

// ---------------------------------------------------------------------------
// Per-format MFMA traits.  A "step" is one MFMA along K.
// ---------------------------------------------------------------------------
template <Kind KD> struct Fmt;

template <> struct Fmt<Kind::F16> {
    static constexpr int ES = 2;            // bytes per element
    static constexpr int STEP_BYTES = 32;   // K bytes per MFMA (32x32x16)
    using Acc = f32x16;
    __device__ static Acc mma(u32x4 a, u32x4 b, Acc c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
};
template <> struct Fmt<Kind::BF16> {
    static constexpr int ES = 2;
    static constexpr int STEP_BYTES = 32;   // 32x32x16
    using Acc = f32x16;
    __device__ static Acc mma(u32x4 a, u32x4 b, Acc c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
};
template <> struct Fmt<Kind::I8> {
    static constexpr int ES = 1;
    static constexpr int STEP_BYTES = 32;   // 32x32x32
    using Acc = i32x16;
    __device__ static Acc mma(u32x4 a, u32x4 b, Acc c) {
        return __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, a),
                                                     __builtin_bit_cast(i32x4, b), c, 0, 0, 0);
    }
};
template <> struct Fmt<Kind::FP8> {
    static constexpr int ES = 1;
    static constexpr int STEP_BYTES = 64;   // 32x32x64, unit (127) E8M0 scales
    using Acc = f32x16;
    // FA, FB: the formats of the first and second operand (the instruction's
    // format fields: 0 E4M3, 1 E5M2)
    template <int FA = 0, int FB = 0>
    __device__ static Acc mma(i32x8 a, i32x8 b, Acc c) {
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FA, FB, 0, 127, 0, 127);
    }
};

// FP8 variants of the kernels: bit 0 A is E5M2, bit 1 B is E5M2, bit 2 one
// scale per row of A and per column of B applied once at the end (otherwise
// the 1 x 128 / 128 x 128 block scales, applied per K block).
constexpr int F8_A_E5M2 = 1, F8_B_E5M2 = 2, F8_ROWS = 4;

// ---------------------------------------------------------------------------
// Tile geometry and LDS layout.
// ---------------------------------------------------------------------------
template <Kind KD, int BM_, int BN_, int WAVES_M_, int WAVES_N_, int KT_BYTES_, int STAGES_>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static constexpr int KT_BYTES = KT_BYTES_;             // bytes of K per K tile
    static constexpr int STAGES = STAGES_;                 // LDS stages (loads run STAGES-1 ahead)
    // register slots of the register-staged path (FP8 keeps one: its wider
    // B tile and block accumulators leave no room for more)
    static constexpr int REG_SLOTS = (KD == Kind::FP8) ? 1 : 3;
    static constexpr int NT = 64 * WAVES_M * WAVES_N;
    static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    static constexpr int TM = WM / 32, TN = WN / 32;       // MFMA tiles per wave
    static constexpr int ES = Fmt<KD>::ES;
    static constexpr int KROWS = KT_BYTES / ES;            // K elements per K tile
    static constexpr int STEPS = KT_BYTES / Fmt<KD>::STEP_BYTES;
    static constexpr int FRAG_BYTES = Fmt<KD>::STEP_BYTES / 2;  // per lane per operand
    static constexpr int CPR_A = KT_BYTES / 16;            // 16-byte chunks per A row
    static constexpr int A_BYTES = BM * KT_BYTES;
    static constexpr int B_ROW = BN * ES;                  // bytes per K row of the B tile
    static constexpr int B_BYTES = KROWS * B_ROW;
    static constexpr int CPR_B = B_ROW / 16;               // 16-byte chunks per B row
    static constexpr int SA_BYTES = (KD == Kind::FP8) ? BM * 4 : 0;   // A-row scales (FP8)
    static constexpr int LDS_BYTES = STAGES * (A_BYTES + B_BYTES + SA_BYTES);
    static constexpr int UA = A_BYTES / 16 / NT;           // 16-byte loads per thread, A
    static constexpr int UB = B_BYTES / 16 / NT;           // 16-byte loads per thread, B
    static_assert(A_BYTES % (16 * NT) == 0 && B_BYTES % (16 * NT) == 0, "staging split");
    static_assert(A_BYTES % 1024 == 0 && B_BYTES % 1024 == 0, "1 KiB load pieces");
    static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile must be 32-aligned");
    static_assert(KT_BYTES == 64 || KT_BYTES == 128, "K tile of 64 or 128 bytes");
    static_assert(STEPS >= 1, "at least one MFMA step per K tile");
    static_assert(KD != Kind::FP8 || KT_BYTES == 128, "FP8: one K tile per 128-wide scale block");
    static_assert(STAGES >= 2 && STAGES <= 5, "2..5 stages");
    static_assert(LDS_BYTES <= 163840, "LDS budget");
};

// A tile: row r (0..BM-1) holds the CPR_A 16-byte chunks of its K bytes; chunk
// c is stored at c ^ swz_a(r).  An MFMA operand read (ds_read_b128) takes one
// chunk from 32 consecutive rows; the swizzle puts rows r..r+7 in 8 distinct
// 16-byte bank slots of a 128-byte bank window and rows r..r+15 in 16
// distinct slots of a 256-byte window.
//   8 chunks per row (128-byte rows): (r & 7) ^ ((r >> 3) & 1)
//   4 chunks per row (64-byte rows, two rows per 128 bytes): ((r >> 1) ^ (r >> 2)) & 3
template <int CPR>
__device__ __forceinline__ uint32_t swz_a(uint32_t r) {
    if constexpr (CPR == 8) return (r & 7u) ^ ((r >> 3) & 1u);
    else return ((r >> 1) ^ (r >> 2)) & 3u;
}

// B tile: K row k holds CPR_B chunks; chunk c is stored at c ^ swz_b(k).
//  16-bit: a transposing read touches 4 consecutive K rows x 2 (or 4) chunks;
//          swz values {0,6,12,10} put them in distinct banks.
//  8-bit:  it touches 8 consecutive K rows x 1 (or 2) chunks; swz = Gray-like
//          (r ^ 2r) spreads them over distinct banks.
template <int ES>
__device__ __forceinline__ uint32_t swz_b(uint32_t k) {
    if constexpr (ES == 2) {
        const uint32_t r = k & 3u;
        return (r ^ (r << 1)) << 1;
    } else {
        const uint32_t r = k & 7u;
        return (r ^ (r << 1)) & 15u;
    }
}

template <class C>
__device__ __forceinline__ uint32_t a_off(uint32_t r, uint32_t c) {
    return r * C::KT_BYTES + ((c ^ swz_a<C::CPR_A>(r)) << 4);
}
template <class C>
__device__ __forceinline__ uint32_t b_off(uint32_t k, uint32_t c) {
    return k * C::B_ROW + ((c ^ swz_b<C::ES>(k)) << 4);
}

// ---------------------------------------------------------------------------
// Workgroup -> output tile.  Workgroups are handed to the 8 XCDs round-robin;
// the first 8*floor(T/8) ids are renumbered so that each XCD receives a
// contiguous run of tiles, and runs are laid out in groups of GROUP_M tile
// rows so an XCD's concurrent tiles share A row panels and B column panels in
// its own L2.
// ---------------------------------------------------------------------------
constexpr int NUM_XCD = 8;
constexpr int GROUP_M = 4;

__device__ __forceinline__ void tile_of(int wg, int tiles_m, int tiles_n, int& tm, int& tn) {
    const int total = tiles_m * tiles_n;
    const int per = total / NUM_XCD;
    int t = wg;
    if (wg < per * NUM_XCD) t = (wg % NUM_XCD) * per + wg / NUM_XCD;
    const int group_size = GROUP_M * tiles_n;
    const int group = t / group_size;
    const int first_m = group * GROUP_M;
    const int gsz = min(tiles_m - first_m, GROUP_M);
    const int in_group = t - group * group_size;
    tm = first_m + in_group % gsz;
    tn = in_group / gsz;
}

// ---------------------------------------------------------------------------
// The kernel.
// ---------------------------------------------------------------------------
struct Stage {
    MPDT_LDS char* A;
    MPDT_LDS char* B;
    MPDT_LDS float* S;   // FP8: per-row A scales of the staged K tile
};

// Workgroup barrier without a memory fence.  (A fence would make the compiler
// drain every direct-to-LDS load in flight, defeating the multi-stage
// pipeline.)  LDS visibility is managed explicitly: a wave waits for its own
// LDS writes (wait_lds) or direct loads (wait_vmem) before the barrier.  The
// signal fences keep the compiler from moving memory accesses across it and
// sched_barrier keeps the scheduler from moving anything across it.
__device__ __forceinline__ void wg_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_sched_barrier(0);
}

// Compile-time loop: f(integral_constant<int, I>) for I in [B, E).
template <int B, int E, class Fn>
__device__ __forceinline__ void static_for(Fn&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

}  // namespace mpdt
