// gemm.hip -- tiled MFMA GEMM for gfx950 (CDNA4): D = A x B + C with FP16 /
// BF16 inputs and FP32 accumulation, INT8 x INT8 -> INT32, and the FP8 E4M3
// GEMM with 1x128 / 128x128 block scales and a BF16 epilogue.
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
// Structure of one workgroup (256 threads = 4 wavefronts, one per SIMD):
//   * WG tile BM x BN of D; wave tile (BM / WAVES_M) x (BN / WAVES_N) held in
//     MFMA accumulators for the whole K loop (acc starts at zero; C is added
//     once in the epilogue).
//   * K is walked in 128-byte tiles (64 FP16/BF16 or 128 INT8/FP8 elements; for
//     FP8 one K tile is exactly one 128-wide scale block).
//   * Global -> registers -> LDS staging with 16-byte loads, two LDS stages,
//     one barrier per K tile; the loads of tile t+2 are in flight while tile
//     t+1 is computed.
//   * LDS layouts are XOR-swizzled in 16-byte chunks.  A (row-major, K
//     contiguous) is read with ds_read_b128 along K; B (row-major, N
//     contiguous) is read with the gfx950 transposing reads ds_read_b64_tr_b16
//     / _b8, which hand each lane one column of a small K x 16 block -- exactly
//     the "column j, consecutive k" operand an MFMA lane needs, so B never has
//     to be transposed in memory.
//   * Edges: loads past M, N or K read zero (bounded 16-byte loads, with an
//     in-register re-alignment for rows that are not 16-byte aligned); stores
//     are masked.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.hpp"
#include "kernels.hpp"

namespace mpdt {

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
    static constexpr int STEP_BYTES = 64;   // 32x32x64, E4M3 x E4M3, unit (127) E8M0 scales
    using Acc = f32x16;
    __device__ static Acc mma(i32x8 a, i32x8 b, Acc c) {
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
    }
};

// ---------------------------------------------------------------------------
// Tile geometry and LDS layout.
// ---------------------------------------------------------------------------
constexpr int KT_BYTES = 128;   // bytes of K per K tile

template <Kind KD, int BM_, int BN_, int WAVES_M_, int WAVES_N_>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static constexpr int NT = 64 * WAVES_M * WAVES_N;
    static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    static constexpr int TM = WM / 32, TN = WN / 32;       // MFMA tiles per wave
    static constexpr int ES = Fmt<KD>::ES;
    static constexpr int KROWS = KT_BYTES / ES;            // K elements per K tile
    static constexpr int STEPS = KT_BYTES / Fmt<KD>::STEP_BYTES;
    static constexpr int FRAG_BYTES = Fmt<KD>::STEP_BYTES / 2;  // per lane per operand
    static constexpr int A_BYTES = BM * KT_BYTES;
    static constexpr int B_ROW = BN * ES;                  // bytes per K row of the B tile
    static constexpr int B_BYTES = KROWS * B_ROW;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int SA_BYTES = (KD == Kind::FP8) ? BM * 4 : 0;
    static constexpr int LDS_BYTES = 2 * STAGE + 2 * SA_BYTES;
    static constexpr int UA = A_BYTES / 16 / NT;           // 16-byte loads per thread, A
    static constexpr int UB = B_BYTES / 16 / NT;           // 16-byte loads per thread, B
    static constexpr int CPR_B = B_ROW / 16;               // 16-byte chunks per B row
    static_assert(A_BYTES % (16 * NT) == 0 && B_BYTES % (16 * NT) == 0, "staging split");
    static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile must be 32-aligned");
    static_assert(LDS_BYTES <= 163840, "LDS budget");
};

// A tile: row r (0..BM-1) holds the 8 16-byte chunks of its 128 K bytes; chunk
// c is stored at c ^ swz_a(r).  Rows r..r+7 of one chunk land in 8 different
// chunks and rows r, r+8 differ too, so the 32-row ds_read_b128 of an MFMA
// operand meets no bank twice in a 128-byte or a 256-byte bank window.
__device__ __forceinline__ uint32_t swz_a(uint32_t r) { return (r & 7u) ^ ((r >> 3) & 1u); }

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

__device__ __forceinline__ uint32_t a_off(uint32_t r, uint32_t c) {
    return r * KT_BYTES + ((c ^ swz_a(r)) << 4);
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
template <Kind KD, class C, bool ALIGNED>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(C::NT / 256, C::NT / 256)))
void gemm_kernel(GemmArgs g) {
    using F = Fmt<KD>;
    using Acc = typename F::Acc;
    constexpr bool IS_FP8 = (KD == Kind::FP8);

    __shared__ __attribute__((aligned(16))) char smem[C::LDS_BYTES];
    MPDT_LDS char* lds = lds_cast(smem);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / C::WAVES_N;
    const int wn = wave % C::WAVES_N;

    int tm, tn;
    tile_of(blockIdx.x, g.tiles_m, g.tiles_n, tm, tn);
    const int m0 = tm * C::BM;
    const int n0 = tn * C::BN;
    const bool full_mn = (m0 + C::BM <= g.M) && (n0 + C::BN <= g.N);

    const int64_t k_bytes = (int64_t)g.K * C::ES;
    const int ntk = (int)((k_bytes + KT_BYTES - 1) / KT_BYTES);

    // ---- staging: which 16-byte chunks this thread moves -------------------
    u32x4 ra[C::UA];
    u32x4 rb[C::UB];
    float rsa = 0.0f;   // FP8: this thread's A-row scale of the staged K tile

    auto load_tile = [&](int kt) {
        const bool full_k = (int64_t)(kt + 1) * KT_BYTES <= k_bytes;
        const int64_t kb0 = (int64_t)kt * KT_BYTES;   // byte offset along K (A) / row base (B)
        if (ALIGNED && full_mn && full_k) {
#pragma unroll
            for (int u = 0; u < C::UA; ++u) {
                const int slot = tid + C::NT * u;
                const int r = slot >> 3, c = slot & 7;
                ra[u] = load16_fast(g.A + (int64_t)(m0 + r) * g.lda_b + kb0 + c * 16);
            }
#pragma unroll
            for (int u = 0; u < C::UB; ++u) {
                const int slot = tid + C::NT * u;
                const int k = slot / C::CPR_B, c = slot % C::CPR_B;
                rb[u] = load16_fast(g.B + (int64_t)(kt * C::KROWS + k) * g.ldb_b +
                                    (int64_t)n0 * C::ES + c * 16);
            }
        } else {
#pragma unroll
            for (int u = 0; u < C::UA; ++u) {
                const int slot = tid + C::NT * u;
                const int r = slot >> 3, c = slot & 7;
                const int row = m0 + r;
                const char* rowp = g.A + (int64_t)row * g.lda_b;
                const char* p = rowp + kb0 + c * 16;
                const char* end = (row < g.M) ? rowp + k_bytes : p;
                ra[u] = load16_row<ALIGNED>(p, end);
            }
#pragma unroll
            for (int u = 0; u < C::UB; ++u) {
                const int slot = tid + C::NT * u;
                const int k = slot / C::CPR_B, c = slot % C::CPR_B;
                const int krow = kt * C::KROWS + k;
                const char* rowp = g.B + (int64_t)krow * g.ldb_b;
                const char* p = rowp + (int64_t)n0 * C::ES + c * 16;
                const char* end = (krow < g.K) ? rowp + (int64_t)g.N * C::ES : p;
                rb[u] = load16_row<ALIGNED>(p, end);
            }
        }
        if constexpr (IS_FP8) {
            if (tid < C::BM) {
                const int row = m0 + tid;
                rsa = (row < g.M) ? g.sA[(int64_t)row * g.ld_sa + kt] : 0.0f;
            }
        }
    };

    auto store_tile = [&](int stage) {
        MPDT_LDS char* As = lds + stage * C::STAGE;
        MPDT_LDS char* Bs = As + C::A_BYTES;
#pragma unroll
        for (int u = 0; u < C::UA; ++u) {
            const int slot = tid + C::NT * u;
            lds_store16(As, a_off(slot >> 3, slot & 7), ra[u]);
        }
#pragma unroll
        for (int u = 0; u < C::UB; ++u) {
            const int slot = tid + C::NT * u;
            lds_store16(Bs, b_off<C>(slot / C::CPR_B, slot % C::CPR_B), rb[u]);
        }
        if constexpr (IS_FP8) {
            if (tid < C::BM) {
                auto sa = (MPDT_LDS float*)(lds + 2 * C::STAGE + stage * C::SA_BYTES);
                sa[tid] = rsa;
            }
        }
    };

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

    auto compute_tile = [&](int stage, int kt) {
        const MPDT_LDS char* As = lds + stage * C::STAGE;
        const MPDT_LDS char* Bs = As + C::A_BYTES;
        Acc blk[IS_FP8 ? C::TM : 1][IS_FP8 ? C::TN : 1];
        if constexpr (IS_FP8) {
#pragma unroll
            for (int i = 0; i < C::TM; ++i)
#pragma unroll
                for (int j = 0; j < C::TN; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) blk[i][j][r] = 0.0f;
        }
#pragma unroll
        for (int s = 0; s < C::STEPS; ++s) {
            // A operand: FRAG_BYTES per lane, along K, from row lrow of each 32-row tile
            u32x4 af[C::TM][C::FRAG_BYTES / 16];
#pragma unroll
            for (int i = 0; i < C::TM; ++i) {
                const uint32_t r = wm * C::WM + i * 32 + lrow;
#pragma unroll
                for (int q = 0; q < C::FRAG_BYTES / 16; ++q) {
                    const uint32_t c = s * (F::STEP_BYTES / 16) + lhalf * (C::FRAG_BYTES / 16) + q;
                    af[i][q] = lds_load16(As, a_off(r, c));
                }
            }
            // B operand: column lrow of each 32-column tile, FRAG_BYTES of K
            u32x2 bf[C::TN][C::FRAG_BYTES / 8];
#pragma unroll
            for (int j = 0; j < C::TN; ++j) {
                const uint32_t col16 = wn * C::WN + j * 32 + 16 * (grp & 1);  // element column
#pragma unroll
                for (int h = 0; h < C::FRAG_BYTES / 8; ++h) {
                    if constexpr (C::ES == 2) {
                        const uint32_t k = s * 16 + 8 * (grp >> 1) + 4 * h + (gp >> 2);
                        const uint32_t c = (col16 >> 3) + ((gp & 3) >> 1);
                        bf[j][h] = lds_read_tr16(Bs, b_off<C>(k, c) + 8 * (gp & 1));
                    } else {
                        const uint32_t k = s * (F::STEP_BYTES) + (C::FRAG_BYTES) * (grp >> 1) +
                                           8 * h + (gp >> 1);
                        const uint32_t c = col16 >> 4;
                        bf[j][h] = lds_read_tr8(Bs, b_off<C>(k, c) + 8 * (gp & 1));
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < C::TM; ++i)
#pragma unroll
                for (int j = 0; j < C::TN; ++j) {
                    if constexpr (IS_FP8) {
                        uint32_t av[8] = {af[i][0][0], af[i][0][1], af[i][0][2], af[i][0][3],
                                          af[i][1][0], af[i][1][1], af[i][1][2], af[i][1][3]};
                        uint32_t bv[8] = {bf[j][0][0], bf[j][0][1], bf[j][1][0], bf[j][1][1],
                                          bf[j][2][0], bf[j][2][1], bf[j][3][0], bf[j][3][1]};
                        i32x8 a, b;
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            a[e] = (int32_t)av[e];
                            b[e] = (int32_t)bv[e];
                        }
                        blk[i][j] = F::mma(a, b, blk[i][j]);
                    } else {
                        u32x4 b = {bf[j][0][0], bf[j][0][1], bf[j][1][0], bf[j][1][1]};
                        acc[i][j] = F::mma(af[i][0], b, acc[i][j]);
                    }
                }
        }
        if constexpr (IS_FP8) {
            // promote the block sums: acc += blk * (sA[row][kb] * sB[kb][n-block])
            const auto sa = (const MPDT_LDS float*)(lds + 2 * C::STAGE + stage * C::SA_BYTES);
            const int nb = (n0 + wn * C::WN) / 128;
            const float sb = (nb < (g.N + 127) / 128) ? g.sB[(int64_t)kt * g.ld_sb + nb] : 0.0f;
#pragma unroll
            for (int i = 0; i < C::TM; ++i) {
                float f[16];
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const uint32_t r = wm * C::WM + i * 32 + 8 * r4 + 4 * lhalf;
                    const u32x4 v = lds_load16((const MPDT_LDS char*)sa, r * 4);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        // (element to scalar first: bit-casting a vector element
                        // directly reads element 0 with this compiler)
                        const uint32_t bits = v[q];
                        f[4 * r4 + q] = __uint_as_float(bits) * sb;
                    }
                }
#pragma unroll
                for (int j = 0; j < C::TN; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[i][j][r] = __builtin_fmaf(blk[i][j][r], f[r], acc[i][j][r]);
            }
        }
    };

    // ---- pipelined K loop ---------------------------------------------------
    if (ntk > 0) {
        load_tile(0);
        store_tile(0);
        if (ntk > 1) load_tile(1);
        __syncthreads();
        for (int kt = 0; kt < ntk; ++kt) {
            const int stage = kt & 1;
            compute_tile(stage, kt);
            if (kt + 1 < ntk) {
                store_tile(stage ^ 1);
                if (kt + 2 < ntk) load_tile(kt + 2);
            }
            __syncthreads();
        }
    }

    // ---- epilogue -----------------------------------------------------------
    // Lane layout of a 32x32 accumulator: column lrow; register r holds row
    // 8*(r/4) + 4*lhalf + (r%4).
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j) {
            const int col = n0 + wn * C::WN + j * 32 + (int)lrow;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm * C::WM + i * 32 + 8 * (r >> 2) + 4 * (int)lhalf + (r & 3);
                if (full_mn || (row < g.M && col < g.N)) {
                    if constexpr (KD == Kind::FP8) {
                        uint16_t* D = (uint16_t*)g.D;
                        D[(int64_t)row * g.ldd + col] = f32_to_bf16_bits(acc[i][j][r]);
                    } else if constexpr (KD == Kind::I8) {
                        int32_t v = acc[i][j][r];
                        if (g.C) v += ((const int32_t*)g.C)[(int64_t)row * g.ldc + col];
                        ((int32_t*)g.D)[(int64_t)row * g.ldd + col] = v;
                    } else {
                        float v = acc[i][j][r];
                        if (g.C) v += ((const float*)g.C)[(int64_t)row * g.ldc + col];
                        ((float*)g.D)[(int64_t)row * g.ldd + col] = v;
                    }
                }
            }
        }
}

// ---------------------------------------------------------------------------
// Host-side launchers (called by the C ABI after validation).
// ---------------------------------------------------------------------------
template <Kind KD, class C>
static hipError_t launch_cfg(const GemmArgs& a0, bool aligned, hipStream_t stream) {
    GemmArgs a = a0;
    a.tiles_m = (a.M + C::BM - 1) / C::BM;
    a.tiles_n = (a.N + C::BN - 1) / C::BN;
    const int64_t tiles = (int64_t)a.tiles_m * a.tiles_n;
    if (tiles == 0) return hipSuccess;
    dim3 grid((unsigned)tiles), block(C::NT);
    if (aligned)
        hipLaunchKernelGGL((gemm_kernel<KD, C, true>), grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((gemm_kernel<KD, C, false>), grid, block, 0, stream, a);
    return hipGetLastError();
}

using CfgF16 = Cfg<Kind::F16, 256, 256, 2, 4>;
using CfgBF16 = Cfg<Kind::BF16, 256, 256, 2, 4>;
using CfgI8 = Cfg<Kind::I8, 256, 256, 2, 4>;
using CfgFP8 = Cfg<Kind::FP8, 128, 256, 2, 4>;

hipError_t launch_gemm(Kind kind, const GemmArgs& a, bool aligned, hipStream_t stream) {
    switch (kind) {
        case Kind::F16: return launch_cfg<Kind::F16, CfgF16>(a, aligned, stream);
        case Kind::BF16: return launch_cfg<Kind::BF16, CfgBF16>(a, aligned, stream);
        case Kind::I8: return launch_cfg<Kind::I8, CfgI8>(a, aligned, stream);
        case Kind::FP8: return launch_cfg<Kind::FP8, CfgFP8>(a, aligned, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace mpdt
