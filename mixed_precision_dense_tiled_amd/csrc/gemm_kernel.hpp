// gemm_kernel.hpp -- the tiled MFMA GEMM kernel template for gfx950 (CDNA4)
// and its launchers, shared by gemm.hip (plain epilogue) and gemm_epi.hip
// (fused bias / activation epilogue): D = A x B + C with FP16 / BF16 inputs
// and FP32 accumulation, INT8 x INT8 -> INT32, and the FP8 E4M3 GEMM with
// 1x128 / 128x128 block scales and a BF16 epilogue.
//
// The operation is the small-matrix multiply-accumulate D = A x B + C of the
// "Tensor Core" chapter of the CUDA advanced handbook ("What a Tensor Core
// does"; FP32 accumulation and scale factors for FP8 in "Precision"), tiled at
// three levels as that chapter draws it (a block owns a tile of C and walks K;
// its warps split the tile; each matrix instruction computes a sub-tile), with
// the improvements its exercise 3 lists (double buffering, larger per-warp
// tiles, conflict-free shared-memory layout).  Everything below is designed
// for CDNA4: 64-lane wavefronts, 32x32 MFMA tiles, a 160 KiB LDS, XCD-local L2.
//
// Two shapes of one kernel template:
//   * one wavefront per SIMD (256 threads, FP16/BF16/INT8 full 256 x 256
//     tiles of an aligned problem): a 128 x 128 wave tile, and a K loop whose
//     program order is written out so the LDS reads of the next MFMA step and
//     the direct loads of later K tiles issue between the MFMAs;
//   * eight wavefronts, two per SIMD (everything else).
// In both:
//   * WG tile BM x BN of D; wave tile (BM / WAVES_M) x (BN / WAVES_N) held in
//     MFMA accumulators for the whole K loop (acc starts at zero; C is added
//     once in the epilogue, except on one-wave full tiles with at least 50 K
//     tiles, where each wave's blocks of C join the accumulators inside the
//     K loop so that C's reads overlap the MFMAs).
//   * K is walked in K tiles of KT_BYTES bytes per row (32 FP16/BF16 or 64
//     INT8 elements; 128 FP8 elements, exactly one scale block).
//   * Interior tiles with 16-byte aligned rows: buffer loads that write LDS
//     directly (no register round trip) fill NS rotating stages, issued
//     NS-1 tiles ahead.
//   * Edge tiles, unaligned rows and the K tail: 16-byte global loads into
//     registers (bounded: bytes past M, N or K read as zero, with an
//     in-register re-alignment for rows that are not 16-byte aligned), then
//     LDS stores; two stages; stores of D are masked.
//   * LDS layouts are XOR-swizzled in 16-byte chunks.  A (row-major, K
//     contiguous) is read with ds_read_b128 along K; B (row-major, N
//     contiguous) is read with the gfx950 transposing reads ds_read_b64_tr_b16
//     / _b8, which hand each lane one column of a small K x 16 block -- exactly
//     the "column j, consecutive k" operand an MFMA lane needs, so B never has
//     to be transposed in memory.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "gemm_common.hpp"

namespace mpdt {

// ---------------------------------------------------------------------------
// The kernel.
// ---------------------------------------------------------------------------
// OUT16 (FP16 / BF16 inputs): D is written in the input format; a separate
// instantiation, so the two output forms are distinct kernels.
// BA (FP16 / BF16 inputs): the fused epilogue -- a bias per output column and
// an activation (GemmArgs::bias, ::act) after C is added (in the epilogue, or
// already inside the K loop).
// exp(y) through the hardware base-2 exponential (about 1 ulp, plus the
// rounding of y log2 e: a relative error near |y| 2^-24).
__device__ __forceinline__ float exp_hw(float y) {
    return __builtin_amdgcn_exp2f(y * 1.4426950408889634f);
}

// erfc(x) for x >= 0: the Chebyshev fit of Press, Teukolsky, Vetterling and
// Flannery ("Numerical Recipes in C", 2nd edition, section 6.2, erfcc), whose
// fractional error is below 1.2e-7 for every x >= 0:
//   t = 1 / (1 + x/2),  erfc(x) = t exp(-x^2 + P(t)),  P a degree-9 polynomial.
// No cancellation anywhere, so the relative accuracy holds deep in the tail.
__device__ __forceinline__ float erfc_nonneg(float x) {
    const float t = __builtin_amdgcn_rcpf(fmaf(0.5f, x, 1.0f));
    float p = 0.17087277f;
    p = fmaf(p, t, -0.82215223f);
    p = fmaf(p, t, 1.48851587f);
    p = fmaf(p, t, -1.13520398f);
    p = fmaf(p, t, 0.27886807f);
    p = fmaf(p, t, -0.18628806f);
    p = fmaf(p, t, 0.09678418f);
    p = fmaf(p, t, 0.37409196f);
    p = fmaf(p, t, 1.00002368f);
    p = fmaf(p, t, -1.26551223f);
    return t * exp_hw(fmaf(-x, x, p));
}

// The fused epilogue's activations in FP32.  GELU: v Phi(v) with
// Phi(v) = erfc(-v / sqrt 2) / 2, taken as v - v erfc(|v| / sqrt 2) / 2 for
// v >= 0 and v erfc(|v| / sqrt 2) / 2 below.  SiLU: v / (1 + exp(-v)) with
// the hardware reciprocal (about 1 ulp).
template <int ACT>
__device__ __forceinline__ float act_apply(float v) {
    if constexpr (ACT == ACT_RELU) {
        return v > 0.0f ? v : 0.0f;
    } else if constexpr (ACT == ACT_GELU) {
        const float h = 0.5f * v * erfc_nonneg(fabsf(v) * 0.70710678118654752f);
        return v >= 0.0f ? v - h : h;
    } else if constexpr (ACT == ACT_SILU) {
        return v * __builtin_amdgcn_rcpf(1.0f + exp_hw(-v));
    } else {
        return v;
    }
}

// F8 (FP8 only): operand formats and the scaling variant (F8_* bits).
template <Kind KD, class C, bool ALIGNED, bool OUT16 = false, bool BA = false, int F8 = 0>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(C::NT / 256, C::NT / 256)))
void gemm_kernel(GemmArgs g) {
    using F = Fmt<KD>;
    using Acc = typename F::Acc;
    constexpr bool IS_FP8 = (KD == Kind::FP8);
    constexpr int FA = (F8 & F8_A_E5M2) ? 1 : 0, FB = (F8 & F8_B_E5M2) ? 1 : 0;
    constexpr bool ROWS = (F8 & F8_ROWS) != 0;   // no block scales in the K loop
    static_assert(F8 == 0 || IS_FP8, "FP8 variants");
    constexpr int NS = C::STAGES;
    constexpr int AHEAD = NS - 1;                 // K tiles loaded ahead of the one computed
    // ONE_WAVE: the interior-tile kernel, one wavefront per SIMD (4 per
    // workgroup) with a 128 x 128 wave tile; its own instruction stream
    // overlaps operand reads and direct loads with its MFMAs.  Otherwise the
    // general kernel (edge tiles, unaligned rows, K tails, FP8).
    constexpr bool ONE_WAVE = !IS_FP8 && C::NT == 256;

    // LDS stages, each its own object, so that the compiler can tell a
    // direct-to-LDS load into one stage from the reads of another.  For FP8
    // the A-row scales of stages 0 and 1 follow their A tiles.
    // One-wave tiles keep their NS stages in one array (stage i at i * STAGE_BYTES,
    // A tile then B tile), so that the stage of a K tile can be a run-time index.
    constexpr int STAGE_BYTES = C::A_BYTES + C::B_BYTES;
    __shared__ __attribute__((aligned(1024))) char sA0[ONE_WAVE ? NS * STAGE_BYTES
                                                                : C::A_BYTES + C::SA_BYTES];
    __shared__ __attribute__((aligned(1024))) char sB0[C::B_BYTES];
    __shared__ __attribute__((aligned(1024))) char sA1[C::A_BYTES + C::SA_BYTES];
    __shared__ __attribute__((aligned(1024))) char sB1[C::B_BYTES];
    __shared__ __attribute__((aligned(NS > 2 ? 1024 : 16))) char sA2[NS > 2 ? C::A_BYTES + C::SA_BYTES : 16];
    __shared__ __attribute__((aligned(NS > 2 ? 1024 : 16))) char sB2[NS > 2 ? C::B_BYTES : 16];
    __shared__ __attribute__((aligned(NS > 3 ? 1024 : 16))) char sA3[NS > 3 ? C::A_BYTES + C::SA_BYTES : 16];
    __shared__ __attribute__((aligned(NS > 3 ? 1024 : 16))) char sB3[NS > 3 ? C::B_BYTES : 16];
    __shared__ __attribute__((aligned(NS > 4 ? 1024 : 16))) char sA4[NS > 4 ? C::A_BYTES + C::SA_BYTES : 16];
    __shared__ __attribute__((aligned(NS > 4 ? 1024 : 16))) char sB4[NS > 4 ? C::B_BYTES : 16];
    // One-wave kernel: each wave's 32 x 32 block of C on its way into the
    // accumulators during the K loop (4 KiB per wave).
    __shared__ __attribute__((aligned(1024))) char sCf[ONE_WAVE ? (C::NT / 64) * 4096 : 16];
    // FP8 keeps the A-row scales of a stage's K tile right after its A tile.
    auto scales_of = [&](char* a) -> MPDT_LDS float* {
        if constexpr (C::SA_BYTES > 0) return (MPDT_LDS float*)(lds_cast(a) + C::A_BYTES);
        else return nullptr;
    };
    // stage(I): the LDS buffers of stage I (a compile-time index, so that
    // every access names its buffer object directly).
    auto stage = [&](auto I) -> Stage {
        constexpr int i = decltype(I)::value;
        if constexpr (ONE_WAVE)
            return {lds_cast(sA0) + i * STAGE_BYTES, lds_cast(sA0) + i * STAGE_BYTES + C::A_BYTES,
                    nullptr};
        else if constexpr (i == 0) return {lds_cast(sA0), lds_cast(sB0), scales_of(sA0)};
        else if constexpr (i == 1) return {lds_cast(sA1), lds_cast(sB1), scales_of(sA1)};
        else if constexpr (i == 2) return {lds_cast(sA2), lds_cast(sB2), scales_of(sA2)};
        else if constexpr (i == 3) return {lds_cast(sA3), lds_cast(sB3), scales_of(sA3)};
        else return {lds_cast(sA4), lds_cast(sB4), scales_of(sA4)};
    };
    // Same with a run-time index (folds to a constant inside unrolled loops).
    auto stage_rt = [&](int i) -> Stage {
        return {i == 0 ? lds_cast(sA0) : i == 1 ? lds_cast(sA1) : i == 2 ? lds_cast(sA2)
                : i == 3 ? lds_cast(sA3) : lds_cast(sA4),
                i == 0 ? lds_cast(sB0) : i == 1 ? lds_cast(sB1) : i == 2 ? lds_cast(sB2)
                : i == 3 ? lds_cast(sB3) : lds_cast(sB4),
                i == 0 ? scales_of(sA0) : i == 1 ? scales_of(sA1) : i == 2 ? scales_of(sA2)
                : i == 3 ? scales_of(sA3) : scales_of(sA4)};
    };
    using I0 = std::integral_constant<int, 0>;

    MPDT_STAMP(0)
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar registers
    const int wm = wave / C::WAVES_N;
    const int wn = wave % C::WAVES_N;

    int tm, tn;
    if (g.int_tm > 0 && g.int_tn > 0) {
        // the interior int_tm x int_tn tiles were launched separately: this
        // grid covers the bottom tile rows, then the right tile columns
        const int bottom = (g.tiles_m - g.int_tm) * g.tiles_n;
        const int b = blockIdx.x;
        if (b < bottom) {
            tm = g.int_tm + b / g.tiles_n;
            tn = b % g.tiles_n;
        } else {
            const int r = b - bottom, cols = g.tiles_n - g.int_tn;
            tm = r / cols;
            tn = g.int_tn + r % cols;
        }
    } else {
        tile_of(blockIdx.x, g.tiles_m, g.tiles_n, tm, tn);
    }
    // (the tile indices come out of VALU integer divisions; taken back to
    // scalar registers here, so that everything derived from them -- the
    // buffer resources of the direct loads above all -- stays scalar)
    const int m0 = __builtin_amdgcn_readfirstlane(tm) * C::BM;
    const int n0 = __builtin_amdgcn_readfirstlane(tn) * C::BN;
    // One-wave kernel: the last tile column of a problem whose B rows end
    // inside a 16-byte chunk is loaded from column N - BN, so that no 16-byte
    // load runs past B's end, and stores only its own columns [n0, N).
    int n0_load = n0;
    if constexpr (ONE_WAVE) {
        if (n0 + C::BN > g.N && ((int64_t)g.N * C::ES) % 16 != 0 && g.N >= C::BN) n0_load = g.N - C::BN;
    }
    const bool full_mn = (m0 + C::BM <= g.M) && (n0 + C::BN <= g.N);

    const int64_t k_bytes = (int64_t)g.K * C::ES;
    const int ntk = (int)((k_bytes + C::KT_BYTES - 1) / C::KT_BYTES);

    // ---- register-staged loads (edge tiles, unaligned rows, K tail) --------
    // A ring of NSLOT register slots (tile t in slot t % NSLOT): the loads of
    // a K tile are issued NSLOT tiles before its data goes to LDS, so their
    // latency hides behind that many tiles of MFMA work.  Slot indices are
    // compile-time constants.
    constexpr int NSLOT = C::REG_SLOTS;
    u32x4 ra[NSLOT][C::UA];
    u32x4 rb[NSLOT][C::UB];
    float rsa[NSLOT];   // FP8: this thread's A-row scale of the staged K tile
#pragma unroll
    for (int q = 0; q < NSLOT; ++q) rsa[q] = 0.0f;

    auto load_scale = [&](int kt, int q) {
        if constexpr (IS_FP8 && !ROWS) {
            if (tid < C::BM) {
                const int row = m0 + tid;
                rsa[q] = (row < g.M) ? g.sA[(int64_t)row * g.ld_sa + kt] : 0.0f;
            }
        }
    };
    auto store_scale = [&](const Stage& s, int q) {
        if constexpr (IS_FP8 && !ROWS) {
            if (tid < C::BM) s.S[tid] = rsa[q];
        }
    };

    auto reg_load = [&](int kt, int q) {
        const int64_t kb0 = (int64_t)kt * C::KT_BYTES;   // byte offset along K (A)
#pragma unroll
        for (int u = 0; u < C::UA; ++u) {
            const int slot = tid + C::NT * u;
            const int r = slot / C::CPR_A, c = slot % C::CPR_A;
            const int row = m0 + r;
            const char* rowp = g.A + (int64_t)row * g.lda_b;
            const char* p = rowp + kb0 + c * 16;
            const char* end = (row < g.M) ? rowp + k_bytes : p;
            ra[q][u] = load16_row<ALIGNED>(p, end);
        }
#pragma unroll
        for (int u = 0; u < C::UB; ++u) {
            const int slot = tid + C::NT * u;
            const int k = slot / C::CPR_B, c = slot % C::CPR_B;
            const int krow = kt * C::KROWS + k;
            const char* rowp = g.B + (int64_t)krow * g.ldb_b;
            const char* p = rowp + (int64_t)n0 * C::ES + c * 16;
            const char* end = (krow < g.K) ? rowp + (int64_t)g.N * C::ES : p;
            rb[q][u] = load16_row<ALIGNED>(p, end);
        }
        load_scale(kt, q);
    };

    auto reg_store = [&](const Stage& s, int q) {
#pragma unroll
        for (int u = 0; u < C::UA; ++u) {
            const int slot = tid + C::NT * u;
            lds_store16(s.A, a_off<C>(slot / C::CPR_A, slot % C::CPR_A), ra[q][u]);
        }
#pragma unroll
        for (int u = 0; u < C::UB; ++u) {
            const int slot = tid + C::NT * u;
            lds_store16(s.B, b_off<C>(slot / C::CPR_B, slot % C::CPR_B), rb[q][u]);
        }
        store_scale(s, q);
    };

    // ---- direct global -> LDS loads (full interior K tiles, aligned rows) ---
    // One wave instruction moves 1 KiB: lane l's 16 bytes land at byte 16*l of
    // the wave's LDS piece.  The swizzle is applied on the global side: the
    // lane that fills physical chunk pc of LDS row r fetches logical chunk
    // pc ^ swz(r) from memory (XOR is its own inverse).  Each wave issues
    // UA + UB of these per K tile.
    // Each load reads through a buffer resource whose wave-uniform base is the
    // K tile's first byte (A: row m0; B: K row kt*KROWS, column n0) and whose
    // range ends at the operand's last byte (the hardware returns zeros for
    // lane offsets past it; the interior-tile conditions keep every read of
    // these paths inside the operand).  Lane offsets (row in the piece times
    // ld, plus the swizzled chunk) are 32-bit and loop-invariant: the swizzles
    // repeat every 16 rows and every wave starts its pieces on a multiple of
    // 16 rows, so they take one or a few registers; piece offsets are scalar.
    // Offsets stay below 2^31 when ld < 2^31 / BM (A) and < 2^31 / KROWS (B).
    // rows per 1 KiB piece and the row periods of the two swizzles
    constexpr int RPA = 1024 / C::KT_BYTES, RPB = 1024 / C::B_ROW;
    constexpr int PERIOD_A = 16, PERIOD_B = C::ES == 2 ? 4 : 8;
    static_assert((C::UA * RPA) % PERIOD_A == 0 && (C::UB * RPB) % PERIOD_B == 0,
                  "each wave's pieces start on a swizzle period");
    const int64_t span_a = (int64_t)(g.M - 1) * g.lda_b + k_bytes;
    const int64_t span_b = (int64_t)(g.K - 1) * g.ldb_b + (int64_t)g.N * C::ES;
    auto tile_rsrc = [](const char* base, int64_t rest) {
        return buffer_rsrc(base, (uint32_t)min(rest, (int64_t)0x7fffffff));
    };
    auto dma16 = [&](const char* base, int64_t rest, MPDT_LDS char* dst, uint32_t voff,
                     uint32_t soff) { buffer_to_lds16(tile_rsrc(base, rest), dst, voff, soff); };
    auto dma_a = [&](int kt, MPDT_LDS char* dst, int wbase, int u) {
        const int lr = lane / C::CPR_A;
        const uint32_t c = (uint32_t)(lane % C::CPR_A) ^ swz_a<C::CPR_A>(u * RPA + lr);
        const int64_t first = (int64_t)m0 * g.lda_b + (int64_t)kt * C::KT_BYTES;
        dma16(g.A + first, span_a - first, dst + (wbase + u) * 1024,
              (uint32_t)lr * (uint32_t)g.lda_b + c * 16u,
              (uint32_t)((wbase + u) * RPA) * (uint32_t)g.lda_b);
    };
    auto dma_b = [&](int kt, MPDT_LDS char* dst, int wbase, int u) {
        const int lr = lane / C::CPR_B;
        const uint32_t c = (uint32_t)(lane % C::CPR_B) ^ swz_b<C::ES>(u * RPB + lr);
        const int64_t first = (int64_t)kt * C::KROWS * g.ldb_b + (int64_t)n0 * C::ES;
        dma16(g.B + first, span_b - first, dst + (wbase + u) * 1024,
              (uint32_t)lr * (uint32_t)g.ldb_b + c * 16u,
              (uint32_t)((wbase + u) * RPB) * (uint32_t)g.ldb_b);
    };
    auto dma_tile = [&](int kt, const Stage& s) {
#pragma unroll
        for (int u = 0; u < C::UA; ++u) dma_a(kt, s.A, wave * C::UA, u);
#pragma unroll
        for (int u = 0; u < C::UB; ++u) dma_b(kt, s.B, wave * C::UB, u);
    };
    constexpr int DMA_PER_TILE = C::UA + C::UB;

    // ---- accumulators -------------------------------------------------------
    Acc acc[C::TM][C::TN];
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

    // lane geometry for operand fetch
    const uint32_t lrow = lane & 31;        // A row / B column within a 32-tile
    const uint32_t lhalf = lane >> 5;       // K half of the MFMA operand
    const uint32_t grp = lane >> 4;         // 16-lane group of a transposing read
    const uint32_t gp = lane & 15;          // lane within that group

    // Operand fragments of one K tile for this wave (all MFMA steps).
    struct Frags {
        u32x4 a[C::STEPS][C::TM][C::FRAG_BYTES / 16];
        u32x2 b[C::STEPS][C::TN][C::FRAG_BYTES / 8];
    };

    auto load_step = [&](const Stage& st, Frags& f, int s) {
        const MPDT_LDS char* As = st.A;
        const MPDT_LDS char* Bs = st.B;
        // A operand: FRAG_BYTES per lane, along K, from row lrow of each 32-row tile
#pragma unroll
        for (int i = 0; i < C::TM; ++i) {
            const uint32_t r = wm * C::WM + i * 32 + lrow;
#pragma unroll
            for (int q = 0; q < C::FRAG_BYTES / 16; ++q) {
                const uint32_t c = s * (F::STEP_BYTES / 16) + lhalf * (C::FRAG_BYTES / 16) + q;
                f.a[s][i][q] = lds_load16(As, a_off<C>(r, c));
            }
        }
        // B operand: column lrow of each 32-column tile, FRAG_BYTES of K
#pragma unroll
        for (int j = 0; j < C::TN; ++j) {
            const uint32_t col16 = wn * C::WN + j * 32 + 16 * (grp & 1);  // element column
#pragma unroll
            for (int h = 0; h < C::FRAG_BYTES / 8; ++h) {
                if constexpr (C::ES == 2) {
                    const uint32_t k = s * 16 + 8 * (grp >> 1) + 4 * h + (gp >> 2);
                    const uint32_t c = (col16 >> 3) + ((gp & 3) >> 1);
                    f.b[s][j][h] = lds_read_tr16(Bs, b_off<C>(k, c) + 8 * (gp & 1));
                } else {
                    const uint32_t k = s * (F::STEP_BYTES) + (C::FRAG_BYTES) * (grp >> 1) +
                                       8 * h + (gp >> 1);
                    const uint32_t c = col16 >> 4;
                    f.b[s][j][h] = lds_read_tr8(Bs, b_off<C>(k, c) + 8 * (gp & 1));
                }
            }
        }
    };

    // MFMAs of one step into `out` (acc, or the FP8 block sums).
    auto mma_step = [&](const Frags& f, int s, Acc (&out)[C::TM][C::TN]) {
        if constexpr (IS_FP8) {
            i32x8 a8[C::TM], b8[C::TN];
#pragma unroll
            for (int i = 0; i < C::TM; ++i)
#pragma unroll
                for (int e = 0; e < 8; ++e) a8[i][e] = (int32_t)f.a[s][i][e >> 2][e & 3];
#pragma unroll
            for (int j = 0; j < C::TN; ++j)
#pragma unroll
                for (int e = 0; e < 8; ++e) b8[j][e] = (int32_t)f.b[s][j][e >> 1][e & 1];
#pragma unroll
            for (int i = 0; i < C::TM; ++i)
#pragma unroll
                for (int j = 0; j < C::TN; ++j) out[i][j] = F::template mma<FA, FB>(a8[i], b8[j], out[i][j]);
        } else {
#pragma unroll
            for (int i = 0; i < C::TM; ++i)
#pragma unroll
                for (int j = 0; j < C::TN; ++j) {
                    const u32x4 b = {f.b[s][j][0][0], f.b[s][j][0][1], f.b[s][j][1][0],
                                     f.b[s][j][1][1]};
                    out[i][j] = F::mma(f.a[s][i][0], b, out[i][j]);
                }
        }
    };

    auto compute_tile = [&](const Stage& st, int kt) {
        Frags f;
        if constexpr (IS_FP8) {
            // All steps' fragments first; then, one 32-row tile at a time, the
            // block sums of its TN tiles (fresh accumulators, 2 MFMAs each)
            // and their promotion, so only TN block accumulators are live.
#pragma unroll
            for (int s = 0; s < C::STEPS; ++s) load_step(st, f, s);
            const int nb = (n0 + wn * C::WN) / 128;
            float sb = 1.0f;
            if constexpr (!ROWS) sb = (nb < (g.N + 127) / 128) ? g.sB[(int64_t)kt * g.ld_sb + nb] : 0.0f;
#pragma unroll
            for (int i = 0; i < C::TM; ++i) {
                Acc blk[C::TN];
#pragma unroll
                for (int j = 0; j < C::TN; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) blk[j][r] = 0.0f;
#pragma unroll
                for (int s = 0; s < C::STEPS; ++s) {
                    i32x8 a8;
#pragma unroll
                    for (int e = 0; e < 8; ++e) a8[e] = (int32_t)f.a[s][i][e >> 2][e & 3];
#pragma unroll
                    for (int j = 0; j < C::TN; ++j) {
                        i32x8 b8;
#pragma unroll
                        for (int e = 0; e < 8; ++e) b8[e] = (int32_t)f.b[s][j][e >> 1][e & 1];
                        blk[j] = F::template mma<FA, FB>(a8, b8, blk[j]);
                    }
                }
                // promote: acc += blk * (sA[row][kb] * sB[kb][n-block])
                // (row-scaled: acc += blk, the scales come at the end)
                float fs[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) fs[r] = 1.0f;
#pragma unroll
                for (int r4 = 0; r4 < 4 && !ROWS; ++r4) {
                    const uint32_t r = wm * C::WM + i * 32 + 8 * r4 + 4 * lhalf;
                    const u32x4 v = lds_load16((const MPDT_LDS char*)st.S, r * 4);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        // (element to scalar first: bit-casting a vector element
                        // directly reads element 0 with this compiler)
                        const uint32_t bits = v[q];
                        fs[4 * r4 + q] = __uint_as_float(bits) * sb;
                    }
                }
#pragma unroll
                for (int j = 0; j < C::TN; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        acc[i][j][r] = __builtin_fmaf(blk[j][r], fs[r], acc[i][j][r]);
            }
        } else {
#pragma unroll
            for (int s = 0; s < C::STEPS; ++s) {
                load_step(st, f, s);
                mma_step(f, s, acc);
            }
        }
    };

    // ---- K loop -------------------------------------------------------------
    // c_folded: C was added to the accumulators inside the K loop (one-wave
    // interior tiles), so the epilogue only writes D.
    bool c_folded = false;
    const bool direct = ALIGNED && full_mn && g.lda_b < (int64_t(1) << 31) / C::BM &&
                        g.ldb_b < (int64_t(1) << 31) / C::KROWS;
    if constexpr (ONE_WAVE) {
        // Launched over every tile of a problem with at least NS K tiles whose
        // operand offsets fit 32 bits (the host checks it; this guard keeps
        // any other problem from being touched).  Rows need only element
        // alignment (16-byte loads from any byte address return the bytes
        // there).  Partial tiles at the M and N edges and a partial last K
        // tile need no separate path: every buffer resource ends at its
        // operand's last byte, so A rows past M and B rows past K read as
        // zero; B columns past N only reach outputs the masked epilogue
        // drops.  A 16-byte load that straddles a resource's end loses all
        // its bytes, so no load may: the last tile column of B is shifted
        // left (n0_load), and the last K tile is read as the KT-byte window
        // that ends on the 16-byte boundary at or after K (each row's end then
        // falls on a chunk boundary); its bytes before the previous tile's end
        // and from K on are cleared in the fragments.
        if (!(k_bytes >= (int64_t)NS * C::KT_BYTES && g.lda_b < (int64_t(1) << 31) / C::BM &&
              g.ldb_b < (int64_t(1) << 31) / C::KROWS && g.ldb_b >= C::B_ROW &&
              (((int64_t)g.N * C::ES) % 16 == 0 || g.N >= C::BN)))
            return;
        if constexpr (ALIGNED && C::STEPS == 2 && C::TM == 4 && C::TN == 4) {
            // One wavefront per SIMD with a 128 x 128 wave tile, at least NS K
            // tiles.  Per K tile t (two MFMA steps):
            //   phase X: the 16 MFMAs of step 0, interleaved with the LDS
            //            reads of step 1's fragments and the set-up of the
            //            direct loads of tile t+NS;
            //   wait for this wave's direct loads of tile t+1 and its LDS
            //   reads, then workgroup barrier B(t+1): tile t+1 is in LDS and
            //   no wave reads tile t's stage any more;
            //   phase Y: the 16 MFMAs of step 1, interleaved with the 8 direct
            //            loads of tile t+NS into tile t's stage and the reads
            //            of tile t+1's step-0 fragments.
            // All NS stages are filled before the loop.  Every K tile issues
            // the same 8 direct loads (past the last tile they read through an
            // empty buffer range: zeros, no memory traffic), so the vmcnt
            // arithmetic is the same everywhere and the loop body is a single
            // block.  The program order written here is pinned by scheduling
            // barriers: a single wave per SIMD issues in order, so whatever
            // sits between two MFMAs is issued while the first one runs.
            static_assert(C::UA == 4 && C::UB == 4, "four A and four B pieces per wave and K tile");
            const int nt = (int)((k_bytes + C::KT_BYTES - 1) / C::KT_BYTES);
            const int last_bytes = (int)(k_bytes - (int64_t)(nt - 1) * C::KT_BYTES);   // 1..KT_BYTES
            const int shift = (16 - last_bytes % 16) % 16;   // the last window starts this far back
            const int64_t kA_last = (int64_t)(nt - 1) * C::KT_BYTES - shift;
            constexpr int WAIT_AHEAD = (NS - 2) * DMA_PER_TILE;   // loads of tiles t+2..t+NS-1
            MPDT_LDS char* const lds0 = lds_cast(sA0);

            // Direct loads.  A piece u (16 rows of the K tile) and B piece u
            // (RPB K rows) of this wave: lane offsets are loop-invariant (the
            // swizzles repeat within a piece pair), scalar offsets per piece;
            // the pieces of one operand share one M0 (piece u adds u KiB
            // through the instruction offset, which also moves the global
            // address, so the scalar offset takes u KiB back off).  The
            // interior-tile conditions keep every live read inside A and B;
            // offsets fit 32 bits (lda < 2^31 / BM, ldb < 2^31 / KROWS).
            const int lra = lane / C::CPR_A, lrb = lane / C::CPR_B;
            const uint32_t voffA = (uint32_t)lra * (uint32_t)g.lda_b +
                                   (((uint32_t)(lane % C::CPR_A) ^ swz_a<C::CPR_A>(lra)) << 4);
            const uint32_t voffB0 = (uint32_t)lrb * (uint32_t)g.ldb_b +
                                    (((uint32_t)(lane % C::CPR_B) ^ swz_b<C::ES>(lrb)) << 4);
            const uint32_t voffB1 = (uint32_t)lrb * (uint32_t)g.ldb_b +
                                    (((uint32_t)(lane % C::CPR_B) ^ swz_b<C::ES>(RPB + lrb)) << 4);
            auto soffA = [&](int u) {
                return (uint32_t)((wave * C::UA + u) * RPA) * (uint32_t)g.lda_b - (uint32_t)u * 1024u;
            };
            auto soffB = [&](int u) {
                return (uint32_t)((wave * C::UB + u) * RPB) * (uint32_t)g.ldb_b - (uint32_t)u * 1024u;
            };
            const uint64_t baseA = (uint64_t)(uintptr_t)g.A + (uint64_t)((int64_t)m0 * g.lda_b);
            const uint64_t baseB = (uint64_t)(uintptr_t)g.B + (uint64_t)((int64_t)n0_load * C::ES);
            const int64_t restA0 = span_a - (int64_t)m0 * g.lda_b;   // bytes of A from baseA
            const int64_t restB0 = span_b - (int64_t)n0_load * C::ES;
            const int64_t stepB = (int64_t)C::KROWS * g.ldb_b;          // bytes per K tile of B
            const int64_t kB_last = ((int64_t)(nt - 1) * C::KROWS - shift / C::ES) * g.ldb_b;
            auto clamp31 = [](int64_t r) { return (uint32_t)(r > 0x7fffffff ? 0x7fffffff : r); };
            // resources of K tile kt (kA = kt * KT_BYTES, kB = kt * stepB)
            auto rsA = [&](int64_t kA, bool live) {
                return rsrc_words(baseA + (uint64_t)kA, live ? clamp31(restA0 - kA) : 0u);
            };
            auto rsB = [&](int64_t kB, bool live) {
                return rsrc_words(baseB + (uint64_t)kB, live ? clamp31(restB0 - kB) : 0u);
            };
            auto dma_piece = [&](auto P, i32x4 ra, i32x4 rb, uint32_t stage_off) {
                constexpr int p = decltype(P)::value;
                // (other instructions sit between the pieces: each keeps the
                // wait state after an M0 write)
                if constexpr (p < C::UA)
                    lds_dma16<p * 1024, true>(ra, lds0 + stage_off + wave * C::UA * 1024, voffA,
                                              soffA(p));
                else
                    lds_dma16<(p - C::UA) * 1024, true>(
                        rb, lds0 + stage_off + C::A_BYTES + wave * C::UB * 1024,
                        (p & 1) ? voffB1 : voffB0, soffB(p - C::UA));
            };

            // Fragment reads.  Lane offsets within a stage: A for step q
            // (tile i adds i*32 rows: the A swizzle repeats every 16 rows);
            // B for column tile j (step q adds QB bytes, half h adds HB: the
            // B swizzle depends only on the K row modulo 4 (16-bit) or 8
            // (8-bit)).
            constexpr uint32_t QB = (C::ES == 2 ? 16 : F::STEP_BYTES) * C::B_ROW;
            constexpr uint32_t HB = (C::ES == 2 ? 4 : 8) * C::B_ROW;
            uint32_t la[2], lb[4];
#pragma unroll
            for (int q = 0; q < 2; ++q)
                la[q] = a_off<C>(wm * C::WM + lrow, q * (F::STEP_BYTES / 16) + lhalf * (C::FRAG_BYTES / 16));
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t col16 = wn * C::WN + j * 32 + 16 * (grp & 1);
                if constexpr (C::ES == 2)
                    lb[j] = C::A_BYTES + b_off<C>(8 * (grp >> 1) + (gp >> 2), (col16 >> 3) + ((gp & 3) >> 1)) +
                            8 * (gp & 1);
                else
                    lb[j] = C::A_BYTES + b_off<C>(C::FRAG_BYTES * (grp >> 1) + (gp >> 1), col16 >> 4) +
                            8 * (gp & 1);
            }
            // read group r (0..6) of step q from the stage at stage_off, in
            // the order the MFMAs consume them: A0+B0, B1, B2, B3, A1, A2, A3
            auto read_group = [&](Frags& f, int q, int r, uint32_t stage_off) {
                auto ra = [&](int i) {
                    f.a[q][i][0] = lds_load16(lds0, stage_off + la[q] + i * 32 * C::KT_BYTES);
                };
                auto rb = [&](int j) {
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const uint32_t o = stage_off + lb[j] + q * QB + h * HB;
                        if constexpr (C::ES == 2) f.b[q][j][h] = lds_read_tr16(lds0, o);
                        else f.b[q][j][h] = lds_read_tr8(lds0, o);
                    }
                };
                if (r == 0) { ra(0); rb(0); }
                else if (r <= 3) rb(r);
                else ra(r - 3);
            };
            auto mma1 = [&](const Frags& f, int q, int idx) {
                const int i = idx / 4, j = idx % 4;
                const u32x4 b = {f.b[q][j][0][0], f.b[q][j][0][1], f.b[q][j][1][0], f.b[q][j][1][1]};
                acc[i][j] = F::mma(f.a[q][i][0], b, acc[i][j]);
            };

            Frags fr;
            // The direct loads of a K tile are split in two halves: its A
            // pieces go out in phase Y of one iteration, its B pieces in
            // phase X of the next (both after the barrier that frees the
            // stage), one per four MFMA slots: a 1 KiB direct load keeps the
            // CU's address unit busy for 16 cycles, and all eight in one
            // phase saturated it and stalled the MFMA stream.  The prologue
            // issues tiles 0..NS-2 whole and tile NS-1's A half; iteration 0
            // issues its B half.
            i32x4 ra_c, rb_c;   // resources of the tile whose B half is due next

            // C inside the K loop.  On a full interior tile with C, C's reads
            // need not wait for the last MFMA: every CU would otherwise read
            // its 256 KiB of C at the same moment after its K loop, with the
            // memory idle before.  Each wave brings its sixteen 32 x 32
            // blocks of C into its own 4 KiB of LDS, one block every c_step K
            // tiles (four 1 KiB direct loads at the end of an iteration), and
            // adds the block to its accumulators in phase Y of the iteration
            // c_step (>= 3) later: by then the block has landed, since the
            // barrier wait of the third iteration after its loads retires
            // every older load of this wave (reads retire in order).  The
            // loads of the next block go out at the end of that iteration,
            // after the block's LDS reads are complete.
            // The sum is taken in a different order than with C added last
            // (C joins after the first partial sums) -- the same FP32 adds
            // otherwise, exact for INT32.
            constexpr int CB = (int)sizeof(typename std::conditional<KD == Kind::I8, int32_t, float>::type);
            const int64_t ldc_b = g.ldc * (int64_t)CB;
            const int c_step = (nt - 2) / 16;
            c_folded = full_mn && g.C != nullptr && c_step >= 3 && ldc_b >= 128 &&
                       ldc_b < (int64_t(1) << 31) / 32;
            MPDT_LDS char* const sCw = lds_cast(sCf) + wave * 4096;
            // lane l of piece u: row 8 u + l / 8 of the block, bytes 16 (l % 8)
            const uint32_t voffC = (uint32_t)(lane >> 3) * (uint32_t)ldc_b + (uint32_t)(lane & 7) * 16u;
            auto c_load = [&](int q) __attribute__((always_inline)) {
                const int64_t row = m0 + wm * C::WM + 32 * (q >> 2), col = n0 + wn * C::WN + 32 * (q & 3);
                const i32x4 rc = rsrc_words((uint64_t)(uintptr_t)g.C + (uint64_t)((row * g.ldc + col) * CB),
                                            (uint32_t)(32 * ldc_b));
                // the previous block's LDS reads have completed before its
                // buffer is refilled
                asm volatile("" ::: "memory");
                wait_lds();
                lds_dma16<0, true>(rc, sCw, voffC, 0u);
                lds_dma16<0, true>(rc, sCw + 1024, voffC, (uint32_t)(8 * ldc_b));
                lds_dma16<0, true>(rc, sCw + 2048, voffC, (uint32_t)(16 * ldc_b));
                lds_dma16<0, true>(rc, sCw + 3072, voffC, (uint32_t)(24 * ldc_b));
            };
            // the wave's block of C from LDS: lane element r is row 8 (r / 4) +
            // 4 lhalf + r % 4, column lrow
            auto c_read = [&](Acc& cv) __attribute__((always_inline)) {
                static_for<0, 16>([&](auto R) __attribute__((always_inline)) {
                    constexpr int r = decltype(R)::value;
                    const uint32_t off = (uint32_t)(8 * (r >> 2) + 4 * (int)lhalf + (r & 3)) * 128u + lrow * 4u;
                    if constexpr (KD == Kind::I8) cv[r] = *(const MPDT_LDS int32_t*)(sCw + off);
                    else cv[r] = *(const MPDT_LDS float*)(sCw + off);
                });
            };
#pragma unroll
            for (int p = 0; p < NS; ++p) {
                const bool lastp = p == nt - 1;
                const i32x4 ra = rsA(lastp ? kA_last : (int64_t)p * C::KT_BYTES, true);
                const i32x4 rb = rsB(lastp ? kB_last : (int64_t)p * stepB, true);
                if (p < NS - 1) {
                    static_for<0, DMA_PER_TILE>([&](auto Q) { dma_piece(Q, ra, rb, p * STAGE_BYTES); });
                } else {
                    static_for<0, C::UA>([&](auto Q) { dma_piece(Q, ra, rb, p * STAGE_BYTES); });
                    ra_c = ra;
                    rb_c = rb;
                }
            }
            wait_vmem<(NS - 2) * DMA_PER_TILE + C::UA>();
            wg_barrier();
#pragma unroll
            for (int r = 0; r < 7; ++r) read_group(fr, 0, r, 0);
            int scur = 0;
            int64_t kA = (int64_t)NS * C::KT_BYTES, kB = (int64_t)NS * stepB;   // tile t+NS
            // One K-loop iteration (K tile t).  FP >= 0: C's block FP, read
            // from LDS at the start of phase Y, joins accumulator tile FP on
            // an MFMA slot of phase Y away from that tile's own MFMA in slot
            // FP (two slots after it for FP < 8, four before it otherwise):
            // the adds then run while other tiles' MFMAs execute.
            auto iter = [&](int t, auto FPc) __attribute__((always_inline)) {
                constexpr int FP = decltype(FPc)::value;
                constexpr int FS = FP < 8 ? FP + 2 : FP - 4;   // first slot of the adds
                Acc cv;
                const int snext = scur + 1 == NS ? 0 : scur + 1;
                const int sprev = scur == 0 ? NS - 1 : scur - 1;   // stage of tile t - 1 + NS
                const uint32_t cur = (uint32_t)scur * STAGE_BYTES;
                const uint32_t nxt = (uint32_t)snext * STAGE_BYTES;
                const uint32_t prv = (uint32_t)sprev * STAGE_BYTES;
                const bool live = t + NS < nt;
                const bool lastl = t + NS == nt - 1;   // the tile loaded now is the last
                i32x4 ra, rb;
                // phase X: the B half of tile t - 1 + NS on slots 9, 11, 13, 15
                static_for<0, 16>([&](auto IDX) {
                    constexpr int idx = decltype(IDX)::value;
                    mma1(fr, 0, idx);
                    if constexpr (idx < 7) read_group(fr, 1, idx, cur);
                    if constexpr (idx == 8) ra = rsA(lastl ? kA_last : kA, live);
                    if constexpr (idx == 10) rb = rsB(lastl ? kB_last : kB, live);
                    if constexpr (idx >= 9 && (idx & 1) == 1)
                        dma_piece(std::integral_constant<int, C::UA + (idx - 9) / 2>{}, ra_c, rb_c, prv);
                    __builtin_amdgcn_sched_barrier(0);
                });
                wait_vmem<WAIT_AHEAD>();
                wait_lds();
                wg_barrier();
                // phase Y: the A half of tile t + NS on slots 0, 4, 8, 12
                static_for<0, 16>([&](auto IDX) {
                    constexpr int idx = decltype(IDX)::value;
                    mma1(fr, 1, idx);
                    if constexpr (FP >= 0) {
                        if constexpr (idx == 0) c_read(cv);
                        if constexpr (idx == FS) acc[FP / C::TN][FP % C::TN] += cv;
                    }
                    if constexpr ((idx & 3) == 0)
                        dma_piece(std::integral_constant<int, idx / 4>{}, ra, rb, cur);
                    else if constexpr ((idx & 1) == 1 && idx / 2 < 7)
                        read_group(fr, 0, idx / 2, nxt);
                    __builtin_amdgcn_sched_barrier(0);
                });
                ra_c = ra;
                rb_c = rb;
                scur = snext;
                kA += C::KT_BYTES;
                kB += stepB;
            };
            if (c_folded) {
                // event q after iteration q * c_step: add block q - 1, load
                // block q; the loop is cut at the events, so each event names
                // its accumulator tile at compile time
                using NoFold = std::integral_constant<int, -1>;
                int t = 0;
                static_for<0, C::TM * C::TN + 1>([&](auto Q) __attribute__((always_inline)) {
                    constexpr int q = decltype(Q)::value;
                    for (; t < q * c_step; ++t) iter(t, NoFold{});
                    iter(t, std::integral_constant<int, q - 1>{});   // (q = 0: no block yet)
                    ++t;
                    if constexpr (q < C::TM * C::TN) {
                        __builtin_amdgcn_sched_barrier(0);
                        c_load(q);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                });
                for (; t < nt - 1; ++t) iter(t, NoFold{});
            } else {
                for (int t = 0; t < nt - 1; ++t) iter(t, std::integral_constant<int, -1>{});
            }
            // last K tile; if it is partial, only the window bytes [shift,
            // shift + last_bytes) are new K: the fragment bytes outside (the
            // previous tile's last bytes, and from K on the next row's bytes,
            // B rows past K or zeros) are cleared in A and in B, so every
            // product outside is exactly zero whatever those bytes hold.  A
            // lane's A fragment of step q covers window bytes [16 c, 16 c + 16),
            // c = 2 q + lhalf; its B fragment half h covers [32 q + 16 lhalf +
            // 8 h, +8), in K order.
            auto keep_n = [](int from, int len, int x) { return min(max(x - from, 0), len); };
            auto mask_a = [&](int q) {
                const int lo = shift, hi = shift + last_bytes;
                const int a0 = 16 * (q * (F::STEP_BYTES / 16) + (int)lhalf * (C::FRAG_BYTES / 16));
                const int b0 = 32 * q + 16 * (int)lhalf;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    fr.a[q][i][0] = mask_head(mask_tail(fr.a[q][i][0], keep_n(a0, 16, hi)), keep_n(a0, 16, lo));
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int h = 0; h < 2; ++h)
                        fr.b[q][j][h] = mask_head8(mask_tail8(fr.b[q][j][h], keep_n(b0 + 8 * h, 8, hi)),
                                                   keep_n(b0 + 8 * h, 8, lo));
            };
            static_assert(F::STEP_BYTES == 32 && C::FRAG_BYTES == 16, "fragment K ranges as above");
            const bool partial = last_bytes < C::KT_BYTES;
            if (partial) mask_a(0);
            const uint32_t cur = (uint32_t)scur * STAGE_BYTES;
            static_for<0, 16>([&](auto IDX) {
                constexpr int idx = decltype(IDX)::value;
                mma1(fr, 0, idx);
                if constexpr (idx < 7) read_group(fr, 1, idx, cur);
                __builtin_amdgcn_sched_barrier(0);
            });
            wait_lds();
            if (partial) mask_a(1);
#pragma unroll
            for (int idx = 0; idx < 16; ++idx) mma1(fr, 1, idx);
            // the empty-range loads of the last tiles still write (zeros) to
            // LDS: let them land before anything else uses it or the wave ends
            wait_vmem<0>();
        }
    } else if (direct) {
        if constexpr (ALIGNED) {
            // Interior tile: full K tiles stream through direct loads issued
            // AHEAD tiles early into NS rotating stages; one barrier per K tile.
            // At the top of iteration kt this wave waits for its own loads of
            // tile kt (leaving the later tiles in flight), then the barrier
            // publishes everyone's loads and retires the reads of tile kt-1,
            // whose stage is refilled with tile kt+AHEAD.
            const int nfull = (int)(k_bytes / C::KT_BYTES);
#pragma unroll
            for (int p = 0; p < AHEAD; ++p)
                if (p < nfull) dma_tile(p, stage_rt(p));
            load_scale(0, 0);
            for (int kt0 = 0; kt0 < nfull; kt0 += NS) {
#pragma unroll
                for (int u = 0; u < NS; ++u) {
                    const int kt = kt0 + u;
                    if (kt < nfull) {
                        const int later = min(AHEAD - 1, nfull - 1 - kt);   // tiles issued after kt
                        if (later >= 2) wait_vmem<2 * DMA_PER_TILE>();
                        else if (later == 1) wait_vmem<DMA_PER_TILE>();
                        else wait_vmem<0>();
                        store_scale(stage_rt(u), 0);
                        wait_lds();
                        wg_barrier();
                        if (kt + AHEAD < nfull)
                            dma_tile(kt + AHEAD, stage_rt((u + AHEAD) % NS));
                        if (kt + 1 < nfull) load_scale(kt + 1, 0);
                        compute_tile(stage_rt(u), kt);
                        wait_lds();
                    }
                }
            }
            if (nfull < ntk) {   // K tail: one partial tile through registers
                reg_load(nfull, 0);
                wait_vmem<0>();
                wg_barrier();   // every wave is past the reads of this stage's last tile
                const Stage sT = stage_rt(nfull % NS);
                reg_store(sT, 0);
                wait_lds();
                wg_barrier();
                compute_tile(sT, nfull);
            }
        }
    } else if (ntk > 0) {
        // Edge tile or rows not 16-byte aligned: guarded loads through the
        // register ring, two LDS stages.  Iteration t computes tile t from
        // stage t % 2, moves tile t+1 from its register slot to the other
        // stage, and issues the loads of tile t+1+NSLOT into that same slot.
        constexpr int UNR = (NSLOT % 2 == 0) ? NSLOT : 2 * NSLOT;   // both indices constant
        reg_load(0, 0);
        reg_store(stage(I0{}), 0);
#pragma unroll
        for (int q = 1; q <= NSLOT; ++q)
            if (q < ntk) reg_load(q, q % NSLOT);
        wait_lds();
        wg_barrier();
        for (int kt0 = 0; kt0 < ntk; kt0 += UNR) {
            static_for<0, UNR>([&](auto U) {
                constexpr int u = decltype(U)::value;
                const int kt = kt0 + u;
                if (kt < ntk) {
                    compute_tile(stage(std::integral_constant<int, u % 2>{}), kt);
                    if (kt + 1 < ntk)
                        reg_store(stage(std::integral_constant<int, (u + 1) % 2>{}), (u + 1) % NSLOT);
                    if (kt + 1 + NSLOT < ntk) reg_load(kt + 1 + NSLOT, (u + 1) % NSLOT);
                    wait_lds();
                    wg_barrier();
                }
            });
        }
    }

    MPDT_STAMP(1)
    // ---- epilogue -----------------------------------------------------------
    // Lane layout of a 32x32 accumulator: column lrow; register r holds row
    // 8*(r/4) + 4*lhalf + (r%4).  D = acc + C in FP32 (INT32), then written in
    // the output format: FP32 / INT32, or FP16 / BF16 (one round to nearest
    // even) for the 16-bit-output entry points; FP8 writes BF16.
    using CT = typename std::conditional<KD == Kind::I8, int32_t, float>::type;
    const CT* const Cp = c_folded ? nullptr : (const CT*)g.C;
    const int row_base = m0 + wm * C::WM + 4 * (int)lhalf;
    const int col_base = n0_load + wn * C::WN + (int)lrow;
    constexpr int NTILE = C::TM * C::TN;
    static_assert(!BA || KD == Kind::F16 || KD == Kind::BF16, "fused epilogue: 16-bit inputs");
    // Fused epilogue: the bias of each of the lane's columns (one per 32-column
    // block; -0 where there is none, since x + (-0) = x for every x), read
    // through a pointer made opaque here, after the K loop, so the loads are
    // not hoisted into it.
    float bcol[BA ? C::TN : 1];
    if constexpr (BA) {
        const float* bptr = g.bias;
        asm volatile("" : "+s"(bptr));
#pragma unroll
        for (int j = 0; j < C::TN; ++j) {
            const int col = col_base + j * 32;
            bcol[j] = (bptr && col < g.N) ? bptr[col] : -0.0f;
        }
    }
    // No activation or ReLU: the store code below, with the bias and the
    // activation in its element conversion.  GELU and SiLU (tens of
    // instructions per element) go through the loop over LDS here instead of
    // code unrolled over all 256 accumulators.
    if constexpr (BA) if (g.act == ACT_GELU || g.act == ACT_SILU) {
        // Fused epilogue, one 32-row block of the wave tile at a time:
        //   (1) v = acc + C, then v = v + bias (FP32 adds, in registers; C of
        //       the next block is read meanwhile), written straight to a
        //       region of LDS of this wave's own (lane-private: 16 bytes per
        //       lane per group of four values);
        //   (2) a loop over that region -- rather than code unrolled over
        //       every register -- applies the activation, rounds once to the
        //       output format and stores D (masked on edge tiles).
        constexpr int PER = C::TN * 16;                  // values per lane per block
        constexpr int REGION = PER * 64 * 4;             // bytes per wave
        static_assert(ONE_WAVE ? (C::NT / 64) * REGION <= NS * STAGE_BYTES
                               : 2 * REGION <= C::A_BYTES && 2 * REGION <= C::B_BYTES,
                      "the blocks fit the K-loop stages");
        MPDT_LDS char* region;
        if constexpr (ONE_WAVE) {
            region = lds_cast(sA0) + wave * REGION;
        } else {
            const int w2 = wave >> 1;
            region = (w2 == 0 ? lds_cast(sA0) : w2 == 1 ? lds_cast(sB0) : w2 == 2 ? lds_cast(sA1)
                                                                                   : lds_cast(sB1)) +
                     (wave & 1) * REGION;
        }
        // (opaque after the K loop, so nothing below is computed early and
        // kept live through it)
        const float* cptr = (const float*)Cp;
        asm volatile("" : "+s"(cptr));
        // (on edge tiles the element is clamped into C: what is read for a
        // position outside M x N is never stored, and every lane issues the
        // same loads without branches)
        auto load_cblk = [&](int i, const float* cp, float (&cv)[PER]) {
            const int rmax = full_mn ? INT_MAX : g.M - 1, cmax = full_mn ? INT_MAX : g.N - 1;
#pragma unroll
            for (int j = 0; j < C::TN; ++j) {
                const int col = min(col_base + j * 32, cmax);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = min(row_base + i * 32 + 8 * (r >> 2) + (r & 3), rmax);
                    cv[j * 16 + r] = cp[(int64_t)row * g.ldc + col];
                }
            }
        };
        using OutT = typename std::conditional<OUT16, uint16_t, float>::type;
        OutT* const Dp = (OutT*)g.D;
        auto finish = [&](int i, auto act_tag) {
            constexpr int ACT = decltype(act_tag)::value;
            // group q: column block j = q / 4, rows 8 (q % 4) + 4 lhalf + 0..3
#pragma unroll 2
            for (int q = 0; q < PER / 4; ++q) {
                const f32x4 v = *(const MPDT_LDS f32x4*)(region + q * 1024 + lane * 16);
                const int row = row_base + i * 32 + 8 * (q & 3);
                const int col = col_base + (q >> 2) * 32;
                OutT* const dp = Dp + (int64_t)row * g.ldd + col;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float a = act_apply<ACT>(v[e]);
                    OutT o;
                    if constexpr (!OUT16) o = a;
                    else if constexpr (KD == Kind::F16) o = f32_to_f16_bits(a);
                    else o = f32_to_bf16_bits(a);
                    if (full_mn || (row + e < g.M && col < g.N && col >= n0)) dp[(int64_t)e * g.ldd] = o;
                }
            }
        };
        float cbuf[2][PER];
        if (cptr) load_cblk(0, cptr, cbuf[0]);
        wg_barrier();   // every wave is done with the K-loop stages
        static_for<0, C::TM>([&](auto I) {
            constexpr int i = decltype(I)::value;
            float (&cur)[PER] = cbuf[i & 1];
            static_for<0, PER / 4>([&](auto Q) {
                constexpr int q = decltype(Q)::value, j = q / 4, r = (q % 4) * 4;
                f32x4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float x = acc[i][j][r + e] + (cptr ? cur[j * 16 + r + e] : 0.0f);
                    v[e] = x + bcol[j];
                }
                *(MPDT_LDS f32x4*)(region + q * 1024 + lane * 16) = v;
            });
            if constexpr (i + 1 < C::TM) {
                if (cptr) {
                    // the next block's reads wait for this block's C: at most
                    // two blocks of C in flight, not every block's at once
                    asm volatile("" : "+s"(cptr) : "v"(cur[0]));
                    load_cblk(i + 1, cptr, cbuf[(i + 1) & 1]);
                }
            }
            if (g.act == ACT_GELU) finish(i, std::integral_constant<int, ACT_GELU>{});   // uniform
            else finish(i, std::integral_constant<int, ACT_SILU>{});
        });
    }
    auto epilogue = [&](auto out_tag, auto act_tag) {
        using OutT = typename decltype(out_tag)::type;
        constexpr int ACT = decltype(act_tag)::value;
        OutT* const Dp = (OutT*)g.D;
        // D's rows start on 128-byte lines (base and pitch)
        const bool d_lines = ((uintptr_t)g.D % 128 == 0) && ((g.ldd * (int64_t)sizeof(OutT)) % 128 == 0);
        // Edge tiles: buffer resources over C and D from the wave's first row
        // (wrow0) to the last element of each (none past M: empty); the
        // buffer form is taken while every range stays below 2^31 bytes and
        // every scalar row offset below 2^30.
        const int wrow0 = m0 + wm * C::WM;
        const int64_t rows_left = (int64_t)g.M - wrow0;
        const int64_t spanD = rows_left > 0 ? ((rows_left - 1) * g.ldd + g.N) * (int64_t)sizeof(OutT) : 0;
        const int64_t spanC = (rows_left > 0 && Cp) ? ((rows_left - 1) * g.ldc + g.N) * (int64_t)sizeof(CT) : 0;
        const bool edge_buf = !full_mn && spanD < (int64_t(1) << 31) && spanC < (int64_t(1) << 31) &&
                              (int64_t)C::WM * g.ldd * (int64_t)sizeof(OutT) < (int64_t(1) << 30) &&
                              (int64_t)C::WM * g.ldc * (int64_t)sizeof(CT) < (int64_t(1) << 30);
        const __amdgpu_buffer_rsrc_t rs_d =
            buffer_rsrc(Dp + (rows_left > 0 ? (int64_t)wrow0 * g.ldd : 0), (uint32_t)(edge_buf ? spanD : 0));
        const __amdgpu_buffer_rsrc_t rs_c =
            buffer_rsrc(Cp ? (const void*)(Cp + (rows_left > 0 ? (int64_t)wrow0 * g.ldc : 0)) : (const void*)Dp,
                        (uint32_t)(edge_buf ? spanC : 0));
        // a: an accumulator element (FP32; INT32 for INT8, kept exact); j:
        // the 32-column block of the wave tile it belongs to
        auto out_val = [&](auto a, CT c, int j) -> OutT {
            if constexpr (KD == Kind::FP8) return f32_to_bf16_bits(a);
            else if constexpr (BA) {
                // v = acc + C, v = v + bias, v = act(v) (none or ReLU): FP32
                // steps, then one rounding to the output format
                float v = a + c;
                v = v + bcol[j];
                v = act_apply<ACT>(v);
                if constexpr (!std::is_same<OutT, uint16_t>::value) return v;
                else if constexpr (KD == Kind::F16) return f32_to_f16_bits(v);
                else return f32_to_bf16_bits(v);
            } else if constexpr (std::is_same<OutT, uint16_t>::value) {
                if constexpr (KD == Kind::F16) return f32_to_f16_bits(a + c);
                else return f32_to_bf16_bits(a + c);
            } else return (OutT)(a + c);
        };
        if constexpr (ONE_WAVE && std::is_same<OutT, uint16_t>::value) {
            if (g.d16_vec && full_mn) {
                // 16-bit D of a one-wave interior tile, staged through LDS so
                // that it leaves in 16-byte stores of whole row segments (the
                // accumulator layout gives each lane one column, so direct
                // stores would be 2 bytes wide).  After a barrier (every wave
                // is done with the K-loop stages) each wave owns a 32 KiB
                // region: its 128 x 128 tile row-major, 256 bytes per row.
                // C is added in FP32 and rounded once, as in the direct form.
                wg_barrier();
                MPDT_LDS char* const reg = lds_cast(sA0) + wave * (C::WM * C::WN * 2);
                static_assert(C::WM * C::WN * 2 * 4 <= NS * STAGE_BYTES, "epilogue staging fits");
                auto ctile = [&](int t) {
                    return Cp + (int64_t)(row_base + (t / C::TN) * 32) * g.ldc + col_base +
                           (t % C::TN) * 32;
                };
                auto load_c = [&](int t, CT (&cv)[16]) {
                    const CT* cp = ctile(t);
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        cv[r] = Cp ? cp[(int64_t)(8 * (r >> 2) + (r & 3)) * g.ldc] : (CT)0;
                };
                auto stage_t = [&](int t, const CT (&cv)[16]) {
                    const int i = t / C::TN, j = t % C::TN;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const uint32_t row = i * 32 + 8 * (r >> 2) + 4 * lhalf + (r & 3);
                        const uint32_t col = j * 32 + lrow;
                        *(MPDT_LDS uint16_t*)(reg + row * (C::WN * 2) + col * 2) =
                            out_val(acc[i][j][r], cv[r], j);
                    }
                };
                CT cbuf[2][16];
                load_c(0, cbuf[0]);
                static_for<0, NTILE>([&](auto T) {
                    constexpr int t = decltype(T)::value;
                    if constexpr (t + 1 < NTILE) load_c(t + 1, cbuf[(t + 1) & 1]);
                    stage_t(t, cbuf[t & 1]);
                });
                // rows of 256 bytes = 16 chunks of 16 bytes; 64 lanes move 4 rows
                constexpr int CPR = C::WN * 2 / 16;
                OutT* const dbase = Dp + (int64_t)(m0 + wm * C::WM) * g.ldd + n0 + wn * C::WN;
#pragma unroll 4
                for (int q = 0; q < C::WM * CPR / 64; ++q) {
                    const int idx = q * 64 + lane;
                    const int row = idx / CPR, c = idx % CPR;
                    const u32x4 v = lds_load16(reg, (uint32_t)(row * (C::WN * 2) + c * 16));
                    u32x4* const dq = reinterpret_cast<u32x4*>(dbase + (int64_t)row * g.ldd + c * 8);
                    if (d_lines) __builtin_nontemporal_store(v, dq);   // (as in the FP32 form below)
                    else *dq = v;
                }
                return;
            }
        }
        if (full_mn) {
            // Interior tile: the wave's 32x32 tiles are written in turn, and C of
            // the next tile is read before this one is stored, so the reads of C
            // stream instead of costing one round trip per element.  (C is either
            // exactly D or disjoint from it -- the C ABI rejects partial overlaps
            // -- so reading C of other elements ahead of these stores is safe.)
            // Row offsets (8*(r/4) + r%4) * ld are wave-uniform.
            auto dtile = [&](int t) {
                return Dp + (int64_t)(row_base + (t / C::TN) * 32) * g.ldd + col_base + (t % C::TN) * 32;
            };
            auto ctile = [&](int t) {
                return Cp + (int64_t)(row_base + (t / C::TN) * 32) * g.ldc + col_base + (t % C::TN) * 32;
            };
            auto load_c = [&](int t, CT (&cv)[16]) {
                const CT* cp = ctile(t);
#pragma unroll
                for (int r = 0; r < 16; ++r) cv[r] = cp[(int64_t)(8 * (r >> 2) + (r & 3)) * g.ldc];
            };
            auto store_t = [&](int t, const CT (&cv)[16]) {
                OutT* dp = dtile(t);
                // D is written once and never read here: with whole 128-byte
                // lines per row segment (D and its row pitch on 128 bytes),
                // non-temporal stores, which keep D from displacing A and B in
                // L2; rows off line boundaries take plain stores (streamed
                // partial lines cost far more than they save)
                if (d_lines) {
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        __builtin_nontemporal_store(out_val(acc[t / C::TN][t % C::TN][r], cv[r], t % C::TN),
                                                    &dp[(int64_t)(8 * (r >> 2) + (r & 3)) * g.ldd]);
                } else {
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        dp[(int64_t)(8 * (r >> 2) + (r & 3)) * g.ldd] =
                            out_val(acc[t / C::TN][t % C::TN][r], cv[r], t % C::TN);
                }
            };
            if (KD != Kind::FP8 && Cp) {
                CT cbuf[2][16];
                load_c(0, cbuf[0]);
                static_for<0, NTILE>([&](auto T) {
                    constexpr int t = decltype(T)::value;
                    if constexpr (t + 1 < NTILE) load_c(t + 1, cbuf[(t + 1) & 1]);
                    store_t(t, cbuf[t & 1]);
                });
            } else {
                CT zero[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) zero[r] = (CT)0;
                static_for<0, NTILE>([&](auto T) { store_t(decltype(T)::value, zero); });
            }
        } else if (edge_buf) {
            // Edge tile through buffer loads and stores, streamed like an
            // interior tile: each resource starts at the wave's first row and
            // ends at the last element of C / D, so rows at or past M fall
            // outside it and the hardware drops their stores (their loads read
            // zero) with no branch; a column outside [n0, N) gets a lane
            // offset of 0xC0000000, far past any range (edge_buf guarantees
            // ranges below 2^31 and scalar offsets below 2^30, so the sum
            // never wraps).  Lane offset: 4 lhalf rows plus the column; scalar
            // offset: the row within the wave tile, wave-uniform.
            constexpr uint32_t OUT_B = sizeof(OutT), C_B = sizeof(CT);
            uint32_t voD[C::TN], voC[C::TN];
#pragma unroll
            for (int j = 0; j < C::TN; ++j) {
                const int col = col_base + j * 32;
                const bool cok = col < g.N && col >= n0;
                voD[j] = cok ? (uint32_t)(4 * (int)lhalf * g.ldd + col) * OUT_B : 0xC0000000u;
                voC[j] = cok ? (uint32_t)(4 * (int)lhalf * g.ldc + col) * C_B : 0xC0000000u;
            }
            // row pitches in bytes, taken to scalar registers: a scalar
            // offset the compiler cannot prove uniform becomes a loop over
            // the lanes' values around every store (edge_buf keeps
            // WM * pitch below 2^30, so 32 bits hold every offset)
            const uint32_t pitch_d = __builtin_amdgcn_readfirstlane((uint32_t)(g.ldd * (int64_t)OUT_B));
            const uint32_t pitch_c = __builtin_amdgcn_readfirstlane((uint32_t)(g.ldc * (int64_t)C_B));
            auto so = [&](int t, int r, uint32_t pitch) {
                return (uint32_t)((t / C::TN) * 32 + 8 * (r >> 2) + (r & 3)) * pitch;
            };
            auto load_c = [&](int t, CT (&cv)[16]) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    if constexpr (KD != Kind::FP8) {
                        const uint32_t bits = __builtin_amdgcn_raw_buffer_load_b32(rs_c, voC[t % C::TN],
                                                                                    so(t, r, pitch_c), 0);
                        cv[r] = __builtin_bit_cast(CT, bits);
                    } else {
                        cv[r] = (CT)0;
                    }
                }
            };
            CT cbuf[2][16];
            load_c(0, cbuf[0]);
            static_for<0, NTILE>([&](auto T) {
                constexpr int t = decltype(T)::value;
                if constexpr (t + 1 < NTILE) load_c(t + 1, cbuf[(t + 1) & 1]);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const OutT o = out_val(acc[t / C::TN][t % C::TN][r], cbuf[t & 1][r], t % C::TN);
                    if constexpr (sizeof(OutT) == 4)
                        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, o), rs_d, voD[t % C::TN],
                                                              so(t, r, pitch_d), 0);
                    else
                        __builtin_amdgcn_raw_buffer_store_b16((uint16_t)o, rs_d, voD[t % C::TN],
                                                              so(t, r, pitch_d), 0);
                }
            });
        } else {
            // Edge tile with offsets too large for the buffer form: every
            // element checked; as above, C of the next 32x32 tile is read
            // (masked) before this one is stored, so the reads are not one
            // round trip per element.
            auto ok = [&](int t, int r) {
                const int row = row_base + (t / C::TN) * 32 + 8 * (r >> 2) + (r & 3);
                const int col = col_base + (t % C::TN) * 32;
                return row < g.M && col < g.N && col >= n0;
            };
            auto at = [&](int t, int r, int64_t ld) {
                return (int64_t)(row_base + (t / C::TN) * 32 + 8 * (r >> 2) + (r & 3)) * ld + col_base +
                       (t % C::TN) * 32;
            };
            auto load_c = [&](int t, CT (&cv)[16]) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    cv[r] = (KD != Kind::FP8 && Cp && ok(t, r)) ? Cp[at(t, r, g.ldc)] : (CT)0;
            };
            CT cbuf[2][16];
            load_c(0, cbuf[0]);
            static_for<0, NTILE>([&](auto T) {
                constexpr int t = decltype(T)::value;
                if constexpr (t + 1 < NTILE) load_c(t + 1, cbuf[(t + 1) & 1]);
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (ok(t, r))
                        Dp[at(t, r, g.ldd)] = out_val(acc[t / C::TN][t % C::TN][r], cbuf[t & 1][r], t % C::TN);
            });
        }
    };
    using Out32 = typename std::conditional<KD == Kind::I8, int32_t, float>::type;
    using OutTag = typename std::conditional<KD == Kind::FP8 || OUT16, std::common_type<uint16_t>,
                                             std::common_type<Out32>>::type;
    if constexpr (IS_FP8 && ROWS) {
        // D = bf16((acc * sA[row]) * sB[col]): ld_sa / ld_sb are the scale
        // vectors' increments (1, or 0 for one scale per tensor)
        static_for<0, NTILE>([&](auto T) {
            constexpr int t = decltype(T)::value;
            const int col = col_base + (t % C::TN) * 32;
            const float sb = col < g.N ? g.sB[(int64_t)col * g.ld_sb] : 0.0f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = row_base + (t / C::TN) * 32 + 8 * (r >> 2) + (r & 3);
                const float sa = row < g.M ? g.sA[(int64_t)row * g.ld_sa] : 0.0f;
                acc[t / C::TN][t % C::TN][r] = (acc[t / C::TN][t % C::TN][r] * sa) * sb;
            }
        });
    }
    if constexpr (BA) {
        if (g.act == ACT_RELU) epilogue(OutTag{}, std::integral_constant<int, ACT_RELU>{});   // uniform
        else if (g.act == ACT_NONE) epilogue(OutTag{}, std::integral_constant<int, ACT_NONE>{});
        // (GELU and SiLU stored D above)
    } else {
        epilogue(OutTag{}, std::integral_constant<int, ACT_NONE>{});
    }
#ifdef MPDT_CLOCK_STAMPS
    __builtin_amdgcn_s_waitcnt(0);   // this wave's stores have completed
    MPDT_STAMP(2)
    if (threadIdx.x == 0 && blockIdx.x < CLOCK_STAMP_WGS) {
        uint64_t* q = g_clock_stamps + blockIdx.x * 6;
        q[0] = stamp_t0; q[1] = stamp_t1; q[2] = stamp_t2;
        q[3] = stamp_r0; q[4] = stamp_r1; q[5] = stamp_r2;
    }
#endif
}

// ---------------------------------------------------------------------------
// The narrow strip at the N edge.  When N is a little over a multiple of the
// 256-column tile (N % 256 in 1..16), the last tile column computes a whole
// tile's K loop for at most 16 useful columns -- on 8191 x 8193 x 4099 one
// extra round of workgroups, a fifth of the run.  Those columns go to this
// kernel instead: a workgroup takes 16 rows (4 per wave) and stages the
// strip of B (K rows x the strip's columns, as FP32, zero past the strip) in
// LDS chunk by chunk; each lane walks K in 16-byte pieces of its rows of A
// and keeps FP32 sums for every row and strip column (FMAs: each product of
// two FP16 / BF16 values is exact in FP32); the wave then adds its lanes'
// sums, and D = acc + C (+ bias, activation) is written as by the tiles.
// ---------------------------------------------------------------------------
constexpr int NSTRIP = 16;        // widest strip taken here
constexpr int STRIP_ROWS = 16;    // rows per workgroup (4 per wave)

template <Kind KD>
__device__ __forceinline__ float half_bits_to_f32(uint32_t b) {
    if constexpr (KD == Kind::F16) return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
    else return __uint_as_float(b << 16);
}

template <Kind KD, bool OUT16, bool BA, int NC>
// (two workgroups per CU: at most 256 registers per lane)
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void gemm_nstrip_kernel(GemmArgs g, int j0) {
    static_assert(KD == Kind::F16 || KD == Kind::BF16, "16-bit inputs");
    // a 64 KiB chunk of the strip; each lane loads all of its 16-byte A
    // pieces of a chunk (PIECES per row) before the first use
    constexpr int STRIP_KC = 16384 / NC;
    constexpr int PIECES = STRIP_KC / 512;
    // row k of the strip starts at float k NC + 4 (k / 8): a lane reads the
    // rows 8 l + e, and the 16 bytes skipped every 8 rows put consecutive
    // lanes on consecutive 16-byte bank groups (conflict-free LDS reads)
    __shared__ __attribute__((aligned(16))) float bs[STRIP_KC * NC + STRIP_KC / 2];
    auto brow_lds = [&](int k) { return &bs[k * NC + (k >> 3) * 4]; };
    const int r = g.N - j0;                       // strip columns, 1..NC
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int i0 = blockIdx.x * STRIP_ROWS + wave * 4;
    const int64_t K = g.K;
    const uint16_t* const B = (const uint16_t*)g.B;
    const int64_t ldb = g.ldb_b / 2;
    const char* arow[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) arow[q] = g.A + (int64_t)(i0 + q < g.M ? i0 + q : 0) * g.lda_b;
    float acc[4][NC];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int c = 0; c < NC; ++c) acc[q][c] = 0.0f;
    for (int64_t k0 = 0; k0 < K; k0 += STRIP_KC) {
        const int kc = (int)(K - k0 < STRIP_KC ? K - k0 : STRIP_KC);
        __syncthreads();                          // the previous chunk's reads are done
        // 8 K elements per piece and row: a full chunk takes plain 16-byte
        // loads (rows need only element alignment: a 16-byte load from any
        // byte address returns the bytes there); the last, partial chunk
        // bounded ones (zeros past K), only for the pieces that reach into it
        u32x4 av[PIECES][4];
        if (kc == STRIP_KC) {
#pragma unroll
            for (int pc = 0; pc < PIECES; ++pc)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    av[pc][q] = *reinterpret_cast<const u32x4*>(arow[q] + (k0 + 8 * lane + 512 * pc) * 2);
        } else {
#pragma unroll
            for (int pc = 0; pc < PIECES; ++pc)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    av[pc][q] = (512 * pc < kc)
                                    ? load16_row<false>(arow[q] + (k0 + 8 * lane + 512 * pc) * 2, arow[q] + K * 2)
                                    : u32x4{0u, 0u, 0u, 0u};
        }
        // Then the strip of B, every load of the chunk issued before the
        // first one is used, so that A's and B's round trips overlap.  B: a
        // thread takes rows tid + 256 it (rows past the chunk read row k0)
        // with one load of NC elements each, which stays inside B on every
        // row but B's last; that row is read as row K - 2 in the batch (no
        // branch between the loads) and element by element beside it, its
        // elements used by the one thread that holds the row.
        // (with K = 1 the batch reads row 0 NC columns to the left of the
        // strip instead -- inside B, since the strip starts at column 256 or
        // later -- and only the last row's own elements are used)
        constexpr int BIT = STRIP_KC / 256;
        uint32_t wb[BIT][NC / 2];
        const int64_t jb = K >= 2 ? j0 : j0 - NC;
#pragma unroll
        for (int it = 0; it < BIT; ++it) {
            const int k = tid + 256 * it;
            int64_t kr = k0 + (k < kc ? k : 0);
            kr = (kr == K - 1 && K >= 2) ? K - 2 : kr;
            const uint16_t* const brow = B + kr * ldb + jb;
            if constexpr (NC == 4) {
                const uint2 x = *reinterpret_cast<const uint2*>(brow);
                wb[it][0] = x.x;
                wb[it][1] = x.y;
            } else {
#pragma unroll
                for (int h = 0; h < NC / 8; ++h) {
                    const u32x4 x = reinterpret_cast<const u32x4*>(brow)[h];
                    wb[it][4 * h] = x[0];
                    wb[it][4 * h + 1] = x[1];
                    wb[it][4 * h + 2] = x[2];
                    wb[it][4 * h + 3] = x[3];
                }
            }
        }
        // B's last row: its r elements, read by every thread (the same
        // addresses for all, no branch); only the thread that holds the row
        // in this chunk uses them
        const int64_t kl = K - 1 - k0;   // its index in the chunk
        const bool own_last = kl < kc && (int)(kl & 255) == tid;
        uint16_t wl[NC];
        {
            const uint16_t* const brow = B + (K - 1) * ldb + j0;
#pragma unroll
            for (int c = 0; c < NC; ++c) wl[c] = brow[c < r ? c : r - 1];
        }
        // the strip of B in LDS as FP32, zeros past K and past the strip
#pragma unroll
        for (int it = 0; it < BIT; ++it) {
            const int k = tid + 256 * it;
            const bool last = own_last && (int)(kl >> 8) == it;
            float v[NC];
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const uint32_t bits = last ? (uint32_t)wl[c] : (wb[it][c >> 1] >> (16 * (c & 1))) & 0xffffu;
                const float x = half_bits_to_f32<KD>(bits);
                v[c] = (k < kc && c < r) ? x : 0.0f;
            }
#pragma unroll
            for (int c4 = 0; c4 < NC / 4; ++c4)
                reinterpret_cast<float4*>(brow_lds(k))[c4] =
                    float4{v[4 * c4], v[4 * c4 + 1], v[4 * c4 + 2], v[4 * c4 + 3]};
        }
        __syncthreads();
#pragma unroll
        for (int pc = 0; pc < PIECES; ++pc) {
            if (512 * pc >= kc) break;            // (the partial chunk's empty pieces)
            const int kk = 8 * lane + 512 * pc;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float b[NC];
#pragma unroll
                for (int c4 = 0; c4 < NC / 4; ++c4) {
                    const float4 v = reinterpret_cast<const float4*>(brow_lds(kk + e))[c4];
                    b[4 * c4] = v.x;
                    b[4 * c4 + 1] = v.y;
                    b[4 * c4 + 2] = v.z;
                    b[4 * c4 + 3] = v.w;
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float a = half_bits_to_f32<KD>((av[pc][q][e >> 1] >> (16 * (e & 1))) & 0xffffu);
#pragma unroll
                    for (int c = 0; c < NC; ++c) acc[q][c] = fmaf(a, b[c], acc[q][c]);
                }
            }
        }
    }
    // the wave's 64 partial sums of every (row, column)
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int m = 32; m >= 1; m >>= 1) acc[q][c] += __shfl_xor(acc[q][c], m, 64);
    // lane c writes column c of the wave's rows: D = acc + C, then the bias and
    // the activation of the fused epilogue, one rounding to the output format
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int i = i0 + q;
        if (i >= g.M) break;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            if (lane != c || c >= r) continue;
            const int j = j0 + c;
            float v = acc[q][c] + (g.C ? ((const float*)g.C)[(int64_t)i * g.ldc + j] : 0.0f);
            if constexpr (BA) {
                if (g.bias) v = v + g.bias[j];
                switch (g.act) {
                    case ACT_RELU: v = act_apply<ACT_RELU>(v); break;
                    case ACT_GELU: v = act_apply<ACT_GELU>(v); break;
                    case ACT_SILU: v = act_apply<ACT_SILU>(v); break;
                    default: break;
                }
            }
            if constexpr (OUT16) {
                ((uint16_t*)g.D)[(int64_t)i * g.ldd + j] =
                    KD == Kind::F16 ? f32_to_f16_bits(v) : f32_to_bf16_bits(v);
            } else {
                ((float*)g.D)[(int64_t)i * g.ldd + j] = v;
            }
        }
    }
}

template <Kind KD, bool OUT16, bool BA>
static hipError_t launch_nstrip(const GemmArgs& a, int j0, hipStream_t stream) {
    const dim3 grid((unsigned)((a.M + STRIP_ROWS - 1) / STRIP_ROWS)), block(256);
    const int r = a.N - j0;
    if (r <= 4) hipLaunchKernelGGL((gemm_nstrip_kernel<KD, OUT16, BA, 4>), grid, block, 0, stream, a, j0);
    else if (r <= 8) hipLaunchKernelGGL((gemm_nstrip_kernel<KD, OUT16, BA, 8>), grid, block, 0, stream, a, j0);
    else hipLaunchKernelGGL((gemm_nstrip_kernel<KD, OUT16, BA, 16>), grid, block, 0, stream, a, j0);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Small FP16 / BF16 / INT8 problems (M, N and K at most 256): the tiled kernels'
// fixed costs -- LDS staging, barriers, a 256 x 256 tile for a few rows --
// set the time there, which is then a chain of memory round trips.  This
// kernel makes it one: a workgroup of four waves takes a 64 x 64 block of D,
// each wave a 32 x 32 block, and every lane issues all of its operand loads
// for the whole of K at once, straight into the MFMA fragments (A: 16 bytes
// of one row per 32x32x16 or 32x32x32 step; B: the same K positions of one
// column, element loads), then runs at most 16 (INT8: 8) MFMAs and the
// epilogue of the tiled kernels (D = acc + C, then the bias and the
// activation, one rounding for 16-bit D; INT8 exact in INT32).  Indices
// past M, N or K are clamped into the operands and their values replaced by
// zero, so no load is guarded by a branch.
// ---------------------------------------------------------------------------
constexpr int SMALL_MAX = 256;     // largest M, N and K taken here

template <Kind KD, bool OUT16, bool BA>
__global__ __launch_bounds__(256) void gemm_small_kernel(GemmArgs g) {
    static_assert(KD == Kind::F16 || KD == Kind::BF16 || KD == Kind::I8, "16-bit or INT8 inputs");
    static_assert(KD != Kind::I8 || (!OUT16 && !BA), "INT8: INT32 D, no fused epilogue");
    using F = Fmt<KD>;
    using E = typename std::conditional<KD == Kind::I8, uint8_t, uint16_t>::type;   // element bits
    using CT = typename std::conditional<KD == Kind::I8, int32_t, float>::type;     // C and D
    constexpr int EPL = 16 / (int)sizeof(E);          // K elements per lane and step
    constexpr int KSTEP = 2 * EPL;                    // K elements per MFMA step
    constexpr int PER_WORD = 4 / (int)sizeof(E);
    constexpr int STEPS = SMALL_MAX / KSTEP;
    constexpr uint32_t EMASK = KD == Kind::I8 ? 0xffu : 0xffffu;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lrow = lane & 31, lhalf = lane >> 5;
    const int i0 = blockIdx.y * 64 + (wave >> 1) * 32;    // the wave's 32 x 32 block
    const int j0 = blockIdx.x * 64 + (wave & 1) * 32;
    const int K = g.K;
    const int ia = i0 + lrow, jb = j0 + lrow;             // this lane's A row, B column
    const E* const arow = (const E*)(g.A + (int64_t)(ia < g.M ? ia : g.M - 1) * g.lda_b);
    const E* const bcol = (const E*)g.B + (jb < g.N ? jb : g.N - 1);
    const int64_t ldb = g.ldb_b / (int64_t)sizeof(E);
    const uint32_t amask = ia < g.M ? ~0u : 0u, bmask = jb < g.N ? EMASK : 0u;

    // step s covers K elements KSTEP s .. KSTEP s + KSTEP - 1; this lane's
    // EPL are KSTEP s + EPL lhalf + e
    u32x4 av[STEPS], bv[STEPS];
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
        const int k = KSTEP * s + EPL * lhalf;
        av[s] = bv[s] = u32x4{0u, 0u, 0u, 0u};
        if (KSTEP * s >= K) continue;
        if (KSTEP * s + KSTEP <= K) {
            av[s] = *reinterpret_cast<const u32x4*>(arow + k) & amask;
        } else {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                uint32_t word = 0;
#pragma unroll
                for (int e = 0; e < PER_WORD; ++e) {
                    const int ke = k + PER_WORD * w + e;
                    word |= (ke < K ? (uint32_t)arow[ke] : 0u) << (8 * sizeof(E) * e);
                }
                av[s][w] = word & amask;
            }
        }
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            uint32_t word = 0;
#pragma unroll
            for (int e = 0; e < PER_WORD; ++e) {
                const int ke = k + PER_WORD * w + e;
                const uint32_t x = bcol[(int64_t)(ke < K ? ke : K - 1) * ldb] & (ke < K ? bmask : 0u);
                word |= x << (8 * sizeof(E) * e);
            }
            bv[s][w] = word;
        }
    }
    typename F::Acc acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0;
#pragma unroll
    for (int s = 0; s < STEPS; ++s)
        if (KSTEP * s < K) acc = F::mma(av[s], bv[s], acc);

    // register r of lane l: row 8 (r / 4) + 4 lhalf + r % 4, column lrow
    const int j = jb;
    if (j >= g.N) return;
    const CT* const Cp = (const CT*)g.C;
    CT cv[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int i = i0 + 8 * (r >> 2) + 4 * lhalf + (r & 3);
        cv[r] = Cp ? Cp[(int64_t)(i < g.M ? i : g.M - 1) * g.ldc + j] : (CT)0;
    }
    float bj = 0.0f;
    if constexpr (BA) bj = g.bias ? g.bias[j] : 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int i = i0 + 8 * (r >> 2) + 4 * lhalf + (r & 3);
        if (i >= g.M) continue;
        auto v = acc[r] + cv[r];
        if constexpr (BA) {
            if (g.bias) v = v + bj;
            switch (g.act) {
                case ACT_RELU: v = act_apply<ACT_RELU>(v); break;
                case ACT_GELU: v = act_apply<ACT_GELU>(v); break;
                case ACT_SILU: v = act_apply<ACT_SILU>(v); break;
                default: break;
            }
        }
        if constexpr (OUT16) {
            ((uint16_t*)g.D)[(int64_t)i * g.ldd + j] = KD == Kind::F16 ? f32_to_f16_bits(v) : f32_to_bf16_bits(v);
        } else {
            ((CT*)g.D)[(int64_t)i * g.ldd + j] = v;
        }
    }
}

template <Kind KD, bool BA>
static hipError_t launch_small(const GemmArgs& a, hipStream_t stream) {
    const dim3 grid((unsigned)((a.N + 63) / 64), (unsigned)((a.M + 63) / 64)), block(256);
    if constexpr (KD == Kind::I8) {
        hipLaunchKernelGGL((gemm_small_kernel<KD, false, false>), grid, block, 0, stream, a);
    } else {
        if (a.out16) hipLaunchKernelGGL((gemm_small_kernel<KD, true, BA>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((gemm_small_kernel<KD, false, BA>), grid, block, 0, stream, a);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Host-side launchers (called by the C ABI after validation).
// ---------------------------------------------------------------------------
template <Kind KD, class C, bool ALIGNED, bool BA, int F8 = 0>
static hipError_t launch_grid(const GemmArgs& a, int64_t tiles, hipStream_t stream) {
    if (tiles <= 0) return hipSuccess;
    if constexpr (KD == Kind::F16 || KD == Kind::BF16) {
        if (a.out16) {
            hipLaunchKernelGGL((gemm_kernel<KD, C, ALIGNED, true, BA>), dim3((unsigned)tiles), dim3(C::NT), 0,
                               stream, a);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((gemm_kernel<KD, C, ALIGNED, false, BA, F8>), dim3((unsigned)tiles), dim3(C::NT), 0,
                       stream, a);
    return hipGetLastError();
}

// General kernel over every tile (or over the edge tiles around an interior
// block launched separately).
template <Kind KD, class C, bool BA = false, int F8 = 0>
static hipError_t launch_general(GemmArgs a, bool aligned, int int_tm, int int_tn,
                                 hipStream_t stream) {
    a.tiles_m = (a.M + C::BM - 1) / C::BM;
    a.tiles_n = (a.N + C::BN - 1) / C::BN;
    a.int_tm = int_tm;
    a.int_tn = int_tn;
    const int64_t tiles = (int64_t)a.tiles_m * a.tiles_n - (int64_t)int_tm * int_tn;
    return aligned ? launch_grid<KD, C, true, BA, F8>(a, tiles, stream)
                   : launch_grid<KD, C, false, BA, F8>(a, tiles, stream);
}

// FP16 / BF16 / INT8: a problem with at least STAGES K tiles (the last may be
// partial) and 32-bit operand offsets goes to the one-wave kernel, edge tiles
// and unaligned rows included (B rows of at least one tile row, and at least
// one full tile column when B's rows end inside a 16-byte chunk); any other
// problem to the general kernel.
template <Kind KD, class C1, class C8, bool BA = false>
static hipError_t launch_mma(const GemmArgs& a0, bool aligned, hipStream_t stream) {
    static_assert(C1::BM == C8::BM && C1::BN == C8::BN, "one tile grid for both kernels");
    if constexpr (KD == Kind::F16 || KD == Kind::BF16 || KD == Kind::I8) {
        if (a0.M <= SMALL_MAX && a0.N <= SMALL_MAX && a0.K <= SMALL_MAX)
            return launch_small<KD, BA>(a0, stream);
    }
    if constexpr (KD == Kind::F16 || KD == Kind::BF16) {
        // a narrow last tile column: the tiles take the whole 256-column
        // blocks, the strip kernel the rest (see gemm_nstrip_kernel)
        const int rem = a0.N % C1::BN;
        if (a0.N > C1::BN && rem >= 1 && rem <= NSTRIP) {
            GemmArgs am = a0;
            am.N = a0.N - rem;
            const hipError_t e = launch_mma<KD, C1, C8, BA>(am, aligned, stream);
            if (e != hipSuccess) return e;
            return a0.out16 ? launch_nstrip<KD, true, BA>(a0, am.N, stream)
                            : launch_nstrip<KD, false, BA>(a0, am.N, stream);
        }
    }
    const int64_t kb = (int64_t)a0.K * C1::ES;
    // (the direct loads' scalar offsets take a piece's instruction offset back
    // off its row offset, which needs rows of at least one B tile row: ldb >=
    // BN elements; lda >= K >= STAGES K tiles covers A)
    const bool one = kb >= (int64_t)C1::STAGES * C1::KT_BYTES && a0.lda_b < (int64_t(1) << 31) / C1::BM &&
                     a0.ldb_b < (int64_t(1) << 31) / C1::KROWS && a0.ldb_b >= C1::B_ROW &&
                     (((int64_t)a0.N * C1::ES) % 16 == 0 || a0.N >= C1::BN);
    if (one) {
        GemmArgs a = a0;
        a.tiles_m = (a0.M + C1::BM - 1) / C1::BM;
        a.tiles_n = (a0.N + C1::BN - 1) / C1::BN;
        a.int_tm = a.int_tn = 0;
        return launch_grid<KD, C1, true, BA>(a, (int64_t)a.tiles_m * a.tiles_n, stream);
    }
    return launch_general<KD, C8, BA>(a0, aligned, 0, 0, stream);
}

// one wavefront per SIMD, interior tiles
template <Kind KD> using Cfg1W = Cfg<KD, 256, 256, 2, 2, 64, 4>;
// eight wavefronts, everything else
template <Kind KD> using Cfg8W = Cfg<KD, 256, 256, 2, 4, 64, 4>;
using CfgFP8 = Cfg<Kind::FP8, 128, 256, 2, 4, 128, 2>;
static_assert(CfgFP8::BM == FP8_TILE_M && CfgFP8::BN == FP8_TILE_N, "one tile grid for both FP8 kernels");

}  // namespace mpdt
