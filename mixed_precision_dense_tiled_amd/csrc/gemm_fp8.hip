// gemm_fp8.hip -- the FP8 E4M3 block-scaled GEMM on full 128 x 256 tiles
// with one wavefront per SIMD (the general kernel in gemm.hip covers edge
// tiles, unaligned rows and K that is not a whole number of scale blocks).
//
// D = sum over 128-wide K blocks of (scale_a[row][kb] * scale_b[kb][col/128])
// times the FP8 block product, accumulated in FP32 and written as BF16: the
// block-scaled FP8 operation of the "Tensor Core" chapter of the CUDA advanced
// handbook ("Precision: FP16, BF16, TF32, FP8": FP8 needs per-row or per-block
// scale factors), the 1 x 128 (A) and 128 x 128 (B) blocks fixed by the C ABI.
//
// Built with MFMA results in VGPRs (-mllvm -amdgpu-mfma-vgpr-form): the block
// sums feed FP32 FMAs every K tile, and VALU instructions cannot read AGPRs.
#include "gemm_common.hpp"

namespace mpdt {

// ---------------------------------------------------------------------------
// FP8 block-scaled GEMM, one wavefront per SIMD, interior tiles.
// ---------------------------------------------------------------------------
// The FP8 path of gemm_kernel (eight wavefronts, 64 x 64 wave tiles, 256
// registers per lane) reads all fragments of a K tile, then runs its MFMAs,
// then rescales the block sums: nothing hides the LDS reads.  Here four
// wavefronts (one per SIMD, 512 registers per lane) each own a 64 x 128 tile
// of the same 128 x 256 workgroup tile (both kernels share one tile grid), so
// the fragments of the next K tile are read, and the block sums of the
// previous one rescaled, while the MFMAs run.
//
// The MFMA operands are swapped: each 32 x 32 block is computed transposed
// (B^T A^T), so all 16 accumulators of a lane belong to one row of D (lane %
// 32) and 16 of its columns.  The scale of a K block is then
// scale_a[row][kb] * scale_b[kb][col / 128] = one multiplier per lane and 32-row
// tile (a wave's 128 columns are one scale block), and the promotion
// acc += blk * (sa * sb) is one FMA per accumulator with no scale table in
// registers.  The operand reads are the same as in gemm_kernel (an MFMA
// operand is "row or column lane % 32, 32 consecutive K bytes" on both sides).
//
// Per K tile t (128 bytes = one scale block = two MFMA steps s0, s1) a wave
// runs 16 MFMA slots in the order s0(i0, j=0..3), s1(i0, j), s0(i1, j),
// s1(i1, j) (i: 32-row tile, j: 32-column tile) with four block accumulators
// blk[j], reused by both row tiles:
//   slots 0-3   promote blk[j] of row tile 1 of K tile t-1, then s0(i0, j);
//   slots 4-7   s1(i0, j); read row tile 1's A fragments and the scales;
//   wait for this wave's direct loads of tile t+1 and its LDS reads, then a
//   workgroup barrier: tile t+1 is in LDS and tile t's stage is free;
//   slots 8-11  promote blk[j] of row tile 0, then s0(i1, j);
//   slots 12-15 s1(i1, j);
//   slots 8-15 also issue the direct loads of tile t+NS into tile t's stage
//   and read tile t+1's fragments for slots 0-7 as their registers free up.
// Every K tile issues the same 14 direct loads per wave (four 1 KiB A pieces,
// eight B pieces, the wave's 64 A-row scales and its B scale); past the last
// tile they read an empty buffer range, so the vmcnt arithmetic never changes
// and the loop body is one basic block whose order scheduling barriers pin.
template <class C>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_fp8_1w_kernel(GemmArgs g) {
    using F = Fmt<Kind::FP8>;
    using Acc = F::Acc;
    static_assert(C::NT == 256 && C::WM == 64 && C::WN == 128 && C::KT_BYTES == 128 &&
                      C::STEPS == 2 && C::UA == 4 && C::UB == 8 && C::B_ROW == 256,
                  "128 x 256 tile, 2 x 2 waves, one 128-byte K tile per scale block");
    constexpr int NS = C::STAGES;
    constexpr int SC_OFF = C::A_BYTES + C::B_BYTES;   // per wave: 256 B A-row scales, 256 B B scale
    constexpr int STAGE_BYTES = SC_OFF + 4 * 512;
    constexpr int DMA_PER_TILE = C::UA + C::UB + 2;
    constexpr int WAIT_AHEAD = (NS - 2) * DMA_PER_TILE;   // loads of tiles t+2..t+NS-1
    static_assert(NS >= 2 && NS * STAGE_BYTES <= 163840, "LDS budget");
    __shared__ __attribute__((aligned(1024))) char lds[NS * STAGE_BYTES];
    MPDT_LDS char* const lds0 = lds_cast(lds);

    MPDT_STAMP(0)
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    int tm, tn;
    tile_of(blockIdx.x, g.tiles_m, g.tiles_n, tm, tn);
    const int m0 = tm * C::BM, n0 = tn * C::BN;
    const int nt = g.K / C::KT_BYTES;
    // (the host launches this kernel over full tiles with whole K tiles only)
    if (m0 + C::BM > g.M || n0 + C::BN > g.N || g.K % C::KT_BYTES != 0 || nt < NS) return;

    const uint32_t lrow = lane & 31, lhalf = lane >> 5, grp = lane >> 4, gp = lane & 15;

    // ---- direct loads -------------------------------------------------------
    // A piece u of this wave: rows (4 wave + u) * 8 .. +7 of the A tile; B piece
    // u: K rows (8 wave + u) * 4 .. +3.  The A swizzle repeats every 16 rows and
    // the B swizzle every 8 K rows, so even and odd pieces have one lane offset
    // each.  Pieces sharing an M0 value move through the instruction offset,
    // which the scalar offset takes back off the global address.
    constexpr int RPA = 1024 / C::KT_BYTES, RPB = 1024 / C::B_ROW;
    const uint32_t lda = (uint32_t)g.lda_b, ldb = (uint32_t)g.ldb_b;
    const int lra = lane / C::CPR_A, lrb = lane / C::CPR_B;
    uint32_t voffA[2], voffB[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        voffA[p] = (uint32_t)lra * lda +
                   (((uint32_t)(lane % C::CPR_A) ^ swz_a<C::CPR_A>(p * RPA + lra)) << 4);
        voffB[p] = (uint32_t)lrb * ldb +
                   (((uint32_t)(lane % C::CPR_B) ^ swz_b<1>(p * RPB + lrb)) << 4);
    }
    // scales: lane l fetches the A-row scale of row (l >> 1) + 32 (l & 1) of the
    // wave's 64 rows, so a lane later finds rows r and r + 32 side by side
    const uint32_t voffSA = (uint32_t)((lane >> 1) + 32 * (lane & 1)) * (uint32_t)g.ld_sa * 4u;
    const uint32_t vzero = 0;
    auto soffA = [&](int u) {
        return (uint32_t)((wave * C::UA + u) * RPA) * lda - (uint32_t)(u & 3) * 1024u;
    };
    auto soffB = [&](int u) {
        return (uint32_t)((wave * C::UB + u) * RPB) * ldb - (uint32_t)(u & 3) * 1024u;
    };
    const int nkb = nt, ncb = (g.N + 127) / 128;
    const int nb = (n0 + wn * C::WN) / 128;
    const uint64_t baseA = (uint64_t)(uintptr_t)g.A + (uint64_t)((int64_t)m0 * g.lda_b);
    const uint64_t baseB = (uint64_t)(uintptr_t)g.B + (uint64_t)n0;
    const int64_t restA0 = ((int64_t)(g.M - 1) * g.lda_b + g.K) - (int64_t)m0 * g.lda_b;
    const int64_t restB0 = ((int64_t)(g.K - 1) * g.ldb_b + g.N) - n0;
    const int64_t stepB = (int64_t)C::KROWS * g.ldb_b;
    const int64_t saFirst = (int64_t)(m0 + wm * C::WM) * g.ld_sa * 4;
    const uint64_t baseSA = (uint64_t)(uintptr_t)g.sA + (uint64_t)saFirst;
    const int64_t restSA0 = ((int64_t)(g.M - 1) * g.ld_sa + nkb) * 4 - saFirst;
    const uint64_t baseSB = (uint64_t)(uintptr_t)g.sB + (uint64_t)nb * 4;
    const int64_t restSB0 = ((int64_t)(nkb - 1) * g.ld_sb + ncb) * 4 - (int64_t)nb * 4;
    const int64_t stepSB = g.ld_sb * 4;
    auto clamp31 = [](int64_t r) { return (uint32_t)(r > 0x7fffffff ? 0x7fffffff : r); };
    struct Rs {
        i32x4 a, b, sa, sb;
    };
    // resources of K tile kt (offsets kt * 128 in A, kt * stepB in B, kt * 4 in
    // the A scales, kt * stepSB in the B scales); a dead tile gets range 0
    auto rs_tile = [&](int64_t kA, int64_t kB, int64_t kSA, int64_t kSB, bool live) -> Rs {
        return {rsrc_words(baseA + (uint64_t)kA, live ? clamp31(restA0 - kA) : 0u),
                rsrc_words(baseB + (uint64_t)kB, live ? clamp31(restB0 - kB) : 0u),
                rsrc_words(baseSA + (uint64_t)kSA, live ? clamp31(restSA0 - kSA) : 0u),
                rsrc_words(baseSB + (uint64_t)kSB, live ? clamp31(restSB0 - kSB) : 0u)};
    };
    auto dma_piece = [&](auto P, const Rs& r, uint32_t stage_off) {
        constexpr int p = decltype(P)::value;
        MPDT_LDS char* const st = lds0 + stage_off;
        if constexpr (p < C::UA) {
            lds_dma16<p * 1024, p == 0>(r.a, st + wave * (C::UA * 1024), voffA[p & 1], soffA(p));
        } else if constexpr (p < C::UA + C::UB) {
            constexpr int u = p - C::UA;   // two M0 groups of four pieces
            lds_dma16<(u & 3) * 1024, (u & 3) == 0>(
                r.b, st + C::A_BYTES + wave * (C::UB * 1024) + (u >> 2) * 4096, voffB[u & 1], soffB(u));
        } else if constexpr (p == C::UA + C::UB) {
            lds_dma4<0, true>(r.sa, st + SC_OFF + wave * 512, voffSA, 0u);
        } else {
            lds_dma4<0, true>(r.sb, st + SC_OFF + wave * 512 + 256, vzero, 0u);
        }
    };

    // ---- fragment reads -----------------------------------------------------
    // A operand (row lrow of a 32-row tile, K bytes 32 lhalf .. +31 of a step):
    // two 16-byte reads; row tile i adds i * 32 rows (a multiple of the swizzle
    // period).  B operand (column lrow of a 32-column tile): four transposing
    // reads of 8 K rows each; step s adds 64 K rows, read h adds 8.
    uint32_t la[2][2], lb[4];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int q = 0; q < 2; ++q)
            la[s][q] = a_off<C>(wm * C::WM + lrow, s * 4 + lhalf * 2 + q);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t col16 = wn * C::WN + j * 32 + 16 * (grp & 1);
        lb[j] = C::A_BYTES + b_off<C>(32 * (grp >> 1) + (gp >> 1), col16 >> 4) + 8 * (gp & 1);
    }
    const uint32_t lsa = SC_OFF + wave * 512 + 8 * lrow;   // rows lrow and lrow + 32
    const uint32_t lsb = SC_OFF + wave * 512 + 256;
    constexpr uint32_t QB = 64 * C::B_ROW, HB = 8 * C::B_ROW;

    struct Fr {
        u32x4 a[2][2][2];   // [row tile][step][16-byte half]
        u32x2 b[2][4][4];   // [step][column tile][8-row read]
    } fr;
    auto rdA = [&](int i, int s, uint32_t so) {
#pragma unroll
        for (int q = 0; q < 2; ++q)
            fr.a[i][s][q] = lds_load16(lds0, so + la[s][q] + (uint32_t)(i * 32 * C::KT_BYTES));
    };
    auto rdB = [&](int s, int j, uint32_t so) {
#pragma unroll
        for (int h = 0; h < 4; ++h) fr.b[s][j][h] = lds_read_tr8(lds0, so + lb[j] + s * QB + h * HB);
    };

    Acc acc[2][4], blk[4];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            acc[0][j][r] = 0.0f;
            acc[1][j][r] = 0.0f;
            blk[j][r] = 0.0f;
        }
    }
    float f[2] = {0.0f, 0.0f};   // sa * sb of the row tiles being promoted
    // slot n's MFMA: step (n >> 2) & 1, row tile n >> 3, column tile n & 3
    auto mfma = [&](int n) {
        const int s = (n >> 2) & 1, i = n >> 3, j = n & 3;
        i32x8 a8, b8;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            a8[e] = (int32_t)fr.a[i][s][e >> 2][e & 3];
            b8[e] = (int32_t)fr.b[s][j][e >> 1][e & 1];
        }
        if (s == 0) {
            const Acc zero = {};
            blk[j] = F::mma(b8, a8, zero);
        } else {
            blk[j] = F::mma(b8, a8, blk[j]);
        }
    };
    auto promote = [&](int i, int j) {
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = __builtin_fmaf(blk[j][r], f[i], acc[i][j][r]);
    };
    u32x2 sap;
    float sbv;
    auto read_scales = [&](uint32_t so) {
        sap = *reinterpret_cast<const MPDT_LDS u32x2*>(lds0 + so + lsa);
        sbv = *reinterpret_cast<const MPDT_LDS float*>(lds0 + so + lsb);
    };
    auto make_f = [&]() {
        const uint32_t s0 = sap[0], s1 = sap[1];
        f[0] = __uint_as_float(s0) * sbv;
        f[1] = __uint_as_float(s1) * sbv;
    };
    // slots 0..7 of a K tile whose stage is at `cur`
    auto phase_x = [&](uint32_t cur) {
        static_for<0, 8>([&](auto N) {
            constexpr int n = decltype(N)::value;
            if constexpr (n < 4) promote(1, n);
            mfma(n);
            if constexpr (n == 0) rdB(1, 3, cur);
            if constexpr (n == 1) rdA(1, 0, cur);
            if constexpr (n == 2) rdA(1, 1, cur);
            if constexpr (n == 4) read_scales(cur);
            if constexpr (n == 7) make_f();
            __builtin_amdgcn_sched_barrier(0);
        });
    };

    // ---- prologue: tiles 0..NS-1 into stages 0..NS-1 ------------------------
    int64_t kA = 0, kB = 0, kSA = 0, kSB = 0;
#pragma unroll
    for (int p = 0; p < NS; ++p) {
        const Rs r = rs_tile(kA, kB, kSA, kSB, true);
        static_for<0, DMA_PER_TILE>([&](auto Q) { dma_piece(Q, r, (uint32_t)(p * STAGE_BYTES)); });
        kA += C::KT_BYTES;
        kB += stepB;
        kSA += 4;
        kSB += stepSB;
    }
    wait_vmem<(NS - 1) * DMA_PER_TILE>();
    wg_barrier();
    // the reads a previous tile's slots 8..15 would have made
    rdA(0, 0, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) rdB(0, j, 0);
    rdA(0, 1, 0);
#pragma unroll
    for (int j = 0; j < 3; ++j) rdB(1, j, 0);

    int scur = 0;
    for (int t = 0; t < nt - 1; ++t) {
        const int snext = scur + 1 == NS ? 0 : scur + 1;
        const uint32_t cur = (uint32_t)scur * STAGE_BYTES;
        const uint32_t nxt = (uint32_t)snext * STAGE_BYTES;
        const Rs rs = rs_tile(kA, kB, kSA, kSB, t + NS < nt);   // tile t+NS
        phase_x(cur);
        wait_vmem<WAIT_AHEAD>();
        wait_lds();
        wg_barrier();
        static_for<8, 16>([&](auto N) {
            constexpr int n = decltype(N)::value;
            if constexpr (n < 12) promote(0, n - 8);
            mfma(n);
            // direct loads of tile t+NS into this tile's stage
            if constexpr (n < 14) {
                dma_piece(std::integral_constant<int, 2 * (n - 8)>{}, rs, cur);
                dma_piece(std::integral_constant<int, 2 * (n - 8) + 1>{}, rs, cur);
            } else {
                dma_piece(std::integral_constant<int, 12 + (n - 14)>{}, rs, cur);
            }
            // tile t+1's fragments for slots 0..7, as their registers free up
            if constexpr (n == 8) rdA(0, 0, nxt);
            if constexpr (n >= 9 && n <= 12) rdB(0, n - 9, nxt);
            if constexpr (n == 13) { rdA(0, 1, nxt); rdB(1, 0, nxt); }
            if constexpr (n == 14) rdB(1, 1, nxt);
            if constexpr (n == 15) rdB(1, 2, nxt);
            __builtin_amdgcn_sched_barrier(0);
        });
        scur = snext;
        kA += C::KT_BYTES;
        kB += stepB;
        kSA += 4;
        kSB += stepSB;
    }
    // last K tile
    phase_x((uint32_t)scur * STAGE_BYTES);
    static_for<8, 16>([&](auto N) {
        constexpr int n = decltype(N)::value;
        if constexpr (n < 12) promote(0, n - 8);
        mfma(n);
        __builtin_amdgcn_sched_barrier(0);
    });
#pragma unroll
    for (int j = 0; j < 4; ++j) promote(1, j);
    // the empty-range loads of the last tiles still write (zeros) to LDS
    wait_vmem<0>();

    MPDT_STAMP(1)
    // ---- epilogue: BF16 D through LDS, 16-byte stores -----------------------
    // A lane holds row i*32 + lrow of the wave tile and, in register 4*r4 + q,
    // column j*32 + 8*r4 + 4*lhalf + q: four consecutive columns per r4, one
    // 8-byte LDS write.  Each wave stages its 64 x 128 tile row-major (256
    // bytes per row, 16-byte chunks XOR-swizzled by row) and writes it out in
    // 16-byte pieces of whole rows.
    wg_barrier();   // every wave is past its reads of the K-tile stages
    MPDT_LDS char* const reg = lds0 + wave * (C::WM * C::WN * 2);
    static_assert(4 * C::WM * C::WN * 2 <= NS * STAGE_BYTES, "epilogue staging fits");
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const uint32_t row = i * 32 + lrow;
                const uint32_t c = j * 4 + r4;
                u32x2 v;
                v[0] = (uint32_t)f32_to_bf16_bits(acc[i][j][4 * r4]) |
                       ((uint32_t)f32_to_bf16_bits(acc[i][j][4 * r4 + 1]) << 16);
                v[1] = (uint32_t)f32_to_bf16_bits(acc[i][j][4 * r4 + 2]) |
                       ((uint32_t)f32_to_bf16_bits(acc[i][j][4 * r4 + 3]) << 16);
                *reinterpret_cast<MPDT_LDS u32x2*>(reg + row * 256 + ((c ^ (row & 15)) << 4) + 8 * lhalf) = v;
            }
    uint16_t* const dbase = (uint16_t*)g.D + (int64_t)(m0 + wm * C::WM) * g.ldd + n0 + wn * C::WN;
#pragma unroll 4
    for (int q = 0; q < C::WM * 16 / 64; ++q) {
        const int idx = q * 64 + lane;
        const int row = idx >> 4, c = idx & 15;
        const u32x4 v = lds_load16(reg, (uint32_t)(row * 256 + ((c ^ (row & 15)) << 4)));
        *reinterpret_cast<u32x4*>(dbase + (int64_t)row * g.ldd + c * 8) = v;
    }
#ifdef MPDT_CLOCK_STAMPS
    __builtin_amdgcn_s_waitcnt(0);
    MPDT_STAMP(2)
    if (threadIdx.x == 0 && blockIdx.x < CLOCK_STAMP_WGS) {
        uint64_t* q = g_clock_stamps + blockIdx.x * 6;
        q[0] = stamp_t0; q[1] = stamp_t1; q[2] = stamp_t2;
        q[3] = stamp_r0; q[4] = stamp_r1; q[5] = stamp_r2;
    }
#endif
}


// one wavefront per SIMD: 128 x 256 tiles, 2 x 2 waves, three stages
using CfgFP8W = Cfg<Kind::FP8, FP8_TILE_M, FP8_TILE_N, 2, 2, 128, 3>;

bool fp8_1w_eligible(const GemmArgs& a, bool aligned) {
    using C = CfgFP8W;
    return aligned && a.K % C::KT_BYTES == 0 && a.K >= C::STAGES * C::KT_BYTES &&
           a.lda_b < (int64_t(1) << 31) / C::BM && a.ldb_b < (int64_t(1) << 31) / C::KROWS &&
           a.ld_sa < (int64_t(1) << 31) / (4 * C::WM) && ((uintptr_t)a.D % 16) == 0 && a.ldd % 8 == 0;
}

hipError_t launch_fp8_1w(const GemmArgs& a0, int tiles_m, int tiles_n, hipStream_t stream) {
    using C = CfgFP8W;
    GemmArgs a = a0;
    a.tiles_m = tiles_m;
    a.tiles_n = tiles_n;
    a.int_tm = a.int_tn = 0;
    hipLaunchKernelGGL((gemm_fp8_1w_kernel<C>), dim3((unsigned)(tiles_m * tiles_n)), dim3(C::NT), 0,
                       stream, a);
    return hipGetLastError();
}

}  // namespace mpdt

#ifdef MPDT_CLOCK_STAMPS
// Stamps of the first n workgroups of the last instrumented launch of the
// one-wave FP8 kernel (same layout as mpdt_clock_stamps).
extern "C" __attribute__((visibility("default"))) int mpdt_clock_stamps_fp8(uint64_t* host, int n) {
    if (n < 0 || n > mpdt::CLOCK_STAMP_WGS) return (int)hipErrorInvalidValue;
    return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(mpdt::g_clock_stamps), (size_t)n * 6 * 8, 0,
                                    hipMemcpyDeviceToHost);
}
#endif
