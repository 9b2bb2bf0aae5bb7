// gemm_fp8.hip -- the FP8 E4M3 block-scaled GEMM on 128 x 256 tiles with one
// wavefront per SIMD (the general kernel in gemm_kernel.hpp covers unaligned
// rows, K that is not a whole number of scale blocks, M below 128 and N not a
// multiple of 16).
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
// FP8 block-scaled GEMM, one wavefront per SIMD.
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
//   slots 4-7   s1(i0, j); read the rest of tile t's fragments;
//   wait for this wave's direct loads of tile t+1 and its LDS reads, then a
//   workgroup barrier: tile t+1 is in LDS and tile t's stage is free;
//   slots 8-11  promote blk[j] of row tile 0, then s0(i1, j);
//   slots 12-15 s1(i1, j);
//   slots 8-15  also read tile t+1's scales and its fragments for slots 0-7,
//               one B column tile per slot as its registers free up.
// The 13 direct loads of tile t+NS (into tile t's stage) go one per slot over
// slots 8-15 of tile t and 0-4 of tile t+1: a 1 KiB direct load keeps the
// CU's address unit busy for 16 cycles, so four waves issuing one per
// 64-cycle MFMA slot stay just below its rate, where bursts stalled the
// issuing waves.  A wave issues one instruction per four cycles and a
// 64-cycle MFMA covers sixteen: the 16 FMAs of a promotion fill the slot they
// sit in, so the LDS reads and scalar work go to the other slots.  The K loop
// is unrolled by the number of stages and LDS holds the A tiles of all
// stages, then the B tiles, then the scales, so every LDS address and M0
// value is a base register or constant plus an immediate.  Every K tile
// issues the same 13 direct loads per wave (four 1 KiB A pieces, eight B
// pieces and one scale load: waves 0 and 1 fetch the A-row scales of rows
// 0-63 and 64-127, waves 2 and 3 the two B scales); past the last tile they
// read an empty buffer range, so the vmcnt arithmetic never changes.
//
// F8 (F8_* bits): E5M2 operands (the MFMA's format fields), or one scale per
// row of A and per column of B instead of the block scales: then every
// promotion multiplier is 1 (the scale loads read an empty range) and the
// scales are applied once, D = bf16((acc * sA[row]) * sB[col]).
template <class C, int F8>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_fp8_1w_kernel(GemmArgs g) {
    using F = Fmt<Kind::FP8>;
    using Acc = F::Acc;
    constexpr int FA = (F8 & F8_A_E5M2) ? 1 : 0, FB = (F8 & F8_B_E5M2) ? 1 : 0;
    constexpr bool ROWS = (F8 & F8_ROWS) != 0;
    static_assert(C::NT == 256 && C::WM == 64 && C::WN == 128 && C::KT_BYTES == 128 &&
                      C::STEPS == 2 && C::UA == 4 && C::UB == 8 && C::B_ROW == 256,
                  "128 x 256 tile, 2 x 2 waves, one 128-byte K tile per scale block");
    constexpr int NS = C::STAGES;
    // LDS: the A tiles of all stages, then their B tiles, then their scale
    // regions (4 x 256 B per stage), so that every fragment read is a base
    // register plus an immediate offset (16 bits).
    constexpr int B_OFF = NS * C::A_BYTES;
    constexpr int S_OFF = B_OFF + NS * C::B_BYTES;
    constexpr int LDS_TOTAL = S_OFF + NS * 1024;
    constexpr int DMA_PER_TILE = C::UA + C::UB + 1;
    constexpr int WAIT_AHEAD = (NS - 2) * DMA_PER_TILE;   // loads of tiles t+2..t+NS-1
    static_assert(NS >= 2 && NS <= 4 && LDS_TOTAL <= 163840, "LDS budget");
    __shared__ __attribute__((aligned(1024))) char lds[LDS_TOTAL];
    MPDT_LDS char* const lds0 = lds_cast(lds);

    MPDT_STAMP(0)
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    int tm, tn;
    tile_of(blockIdx.x, g.tiles_m, g.tiles_n, tm, tn);
    // Edge tiles: the last row tile of a problem whose M is not a multiple of
    // 128 moves up to end at row M - 1 (M >= 128; rows it shares with the tile
    // above are computed twice and stored once, from row_lo on); columns past
    // N read zeros (masked B loads) and are not stored.
    const int row_lo = __builtin_amdgcn_readfirstlane(tm) * C::BM;
    const int m0 = min(row_lo, g.M - C::BM), n0 = __builtin_amdgcn_readfirstlane(tn) * C::BN;
    const int nt = g.K / C::KT_BYTES;
    // (the host launches this kernel with M >= 128 and whole K tiles only)
    if (m0 < 0 || g.K % C::KT_BYTES != 0 || nt < NS) return;

    const uint32_t lrow = lane & 31, lhalf = lane >> 5, grp = lane >> 4, gp = lane & 15;

    // ---- direct loads -------------------------------------------------------
    // A piece u of this wave: rows (4 wave + u) * 8 .. +7 of the A tile; B piece
    // u: K rows (8 wave + u) * 4 .. +3.  The A swizzle repeats every 16 rows and
    // the B swizzle every 8 K rows, so even and odd pieces have one lane offset
    // each.  Pieces sharing an M0 value move through the instruction offset,
    // which the scalar offset takes back off the global address.  Each buffer
    // resource starts at the K tile's first byte and spans the bytes the tile
    // reads, or nothing past the last tile.  A lane whose 16 B columns lie at
    // or past N gets a lane offset of 2^31, past every range (whether or not
    // the range check counts the scalar offset): it reads zeros and touches
    // no memory.  N is a multiple of 16 here, so a chunk is all in or all out.
    constexpr int RPA = 1024 / C::KT_BYTES, RPB = 1024 / C::B_ROW;
    const uint32_t lda = (uint32_t)g.lda_b, ldb = (uint32_t)g.ldb_b;
    const int lra = lane / C::CPR_A, lrb = lane / C::CPR_B;
    uint32_t voffA[2], voffB[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        voffA[p] = (uint32_t)lra * lda +
                   (((uint32_t)(lane % C::CPR_A) ^ swz_a<C::CPR_A>(p * RPA + lra)) << 4);
        const uint32_t gc = (uint32_t)(lane % C::CPR_B) ^ swz_b<1>(p * RPB + lrb);
        voffB[p] = (int)(gc * 16) < g.N - n0 ? (uint32_t)lrb * ldb + (gc << 4) : 0x80000000u;
    }
    auto soffA = [&](int u) __attribute__((always_inline)) {
        return (uint32_t)((wave * C::UA + u) * RPA) * lda - (uint32_t)(u & 3) * 1024u;
    };
    auto soffB = [&](int u) __attribute__((always_inline)) {
        return (uint32_t)((wave * C::UB + u) * RPB) * ldb - (uint32_t)(u & 3) * 1024u;
    };
    const uint32_t rangeA = (uint32_t)(C::BM - 1) * lda + C::KT_BYTES;
    // (+4 KiB: every live lane's offset stays inside the range also when the
    // check leaves out the scalar offset and B rows are narrow)
    const uint32_t rangeB = (uint32_t)(C::KROWS - 1) * ldb + C::B_ROW + 4096u;
    const uint64_t baseA = (uint64_t)(uintptr_t)g.A + (uint64_t)((int64_t)m0 * g.lda_b);
    const uint64_t baseB = (uint64_t)(uintptr_t)g.B + (uint64_t)n0;
    const uint64_t stepB = (uint64_t)C::KROWS * (uint64_t)g.ldb_b;
    // Scale loads (one per wave and K tile, 64 lanes into the wave's 256-byte
    // region of the stage).  Waves 0, 1: A-row scales of rows 64 w .. 64 w + 63,
    // lane l taking row (l >> 1) + 32 (l & 1), so that rows q and q + 32 sit
    // side by side.  Waves 2, 3: the B scales of the tile's two 128-column
    // blocks, lane l taking block l & 1.
    const bool scaleA = wave < 2;
    const uint32_t ldsa4 = (uint32_t)g.ld_sa * 4u;
    const uint32_t voffS = scaleA ? (uint32_t)((lane >> 1) + 32 * (lane & 1)) * ldsa4
                                  : (uint32_t)(lane & 1) * 4u;
    const uint32_t rangeS = ROWS ? 0u : scaleA ? 63u * ldsa4 + 4u : (n0 + 128 < g.N ? 8u : 4u);
    const uint64_t baseS = scaleA ? (uint64_t)(uintptr_t)g.sA + (uint64_t)((int64_t)(m0 + wave * 64) * ldsa4)
                            : (uint64_t)(uintptr_t)g.sB + (uint64_t)(n0 / 128) * 4u;
    const uint64_t stepS = scaleA ? 4u : (uint64_t)g.ld_sb * 4u;
    // Resources of the next K tile to load, advanced in place (the base
    // address stays below 2^48, so its high word never reaches the stride
    // field); a dead tile (past the last) gets range 0.
    struct Rs {
        i32x4 a, b, s;
    };
    Rs rs = {rsrc_words(baseA, rangeA), rsrc_words(baseB, rangeB), rsrc_words(baseS, rangeS)};
    auto bump = [](i32x4& r, uint64_t step) __attribute__((always_inline)) {
        const uint64_t b = ((uint64_t)(uint32_t)r[1] << 32 | (uint32_t)r[0]) + step;
        r[0] = (int32_t)(uint32_t)b;
        r[1] = (int32_t)(uint32_t)(b >> 32);
    };
    auto rs_next = [&](bool live) __attribute__((always_inline)) {
        bump(rs.a, C::KT_BYTES);
        bump(rs.b, stepB);
        bump(rs.s, stepS);
        rs.a[2] = live ? (int32_t)rangeA : 0;
        rs.b[2] = live ? (int32_t)rangeB : 0;
        rs.s[2] = live ? (int32_t)rangeS : 0;
    };
    auto dma_piece = [&](auto P, const Rs& r, auto STG) __attribute__((always_inline)) {
        constexpr int p = decltype(P)::value, S = decltype(STG)::value;
        if constexpr (p < C::UA) {
            lds_dma16<p * 1024, p == 0>(r.a, lds0 + S * C::A_BYTES + wave * (C::UA * 1024), voffA[p & 1],
                                        soffA(p));
        } else if constexpr (p < C::UA + C::UB) {
            constexpr int u = p - C::UA;   // two M0 groups of four pieces
            lds_dma16<(u & 3) * 1024, (u & 3) == 0>(
                r.b, lds0 + B_OFF + S * C::B_BYTES + wave * (C::UB * 1024) + (u >> 2) * 4096,
                voffB[u & 1], soffB(u));
        } else {
            lds_dma4<0, true>(r.s, lds0 + S_OFF + S * 1024 + wave * 256, voffS, 0u);
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
        lb[j] = B_OFF + b_off<C>(32 * (grp >> 1) + (gp >> 1), col16 >> 4) + 8 * (gp & 1);
    }
    const uint32_t lsa = S_OFF + wm * 256 + 8 * lrow;      // A-row scales of rows lrow, lrow + 32
    const uint32_t lsb = S_OFF + 2 * 256 + 4 * wn;         // this wave's B scale
    constexpr uint32_t QB = 64 * C::B_ROW, HB = 8 * C::B_ROW;
    static_assert(C::B_BYTES + QB + 3 * HB < 65536, "16-bit read offsets");

    struct Fr {
        u32x4 a[2][2][2];   // [row tile][step][16-byte half]
        u32x2 b[2][4][4];   // [step][column tile][8-row read]
    } fr;
    auto rdA = [&](int i, int s, auto STG) __attribute__((always_inline)) {
        constexpr uint32_t so = decltype(STG)::value * C::A_BYTES;
#pragma unroll
        for (int q = 0; q < 2; ++q)
            fr.a[i][s][q] = lds_load16(lds0, la[s][q] + so + (uint32_t)(i * 32 * C::KT_BYTES));
    };
    auto rdB = [&](int s, int j, auto STG) __attribute__((always_inline)) {
        // A stage past the 16-bit immediate range moves the base once per
        // call (kept opaque, so the compiler does not fold it back into four
        // separate adds).
        constexpr uint32_t so = decltype(STG)::value * C::B_BYTES;
        constexpr uint32_t hi = (so + QB + 3 * HB) >= 65536u ? 65536u : 0u;
        uint32_t base = lb[j];
        if constexpr (hi != 0) {
            base += hi;
            asm volatile("" : "+v"(base));
        }
#pragma unroll
        for (int h = 0; h < 4; ++h) fr.b[s][j][h] = lds_read_tr8(lds0, base + (so - hi) + s * QB + h * HB);
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
    auto mfma = [&](int n) __attribute__((always_inline)) {
        const int s = (n >> 2) & 1, i = n >> 3, j = n & 3;
        i32x8 a8, b8;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            a8[e] = (int32_t)fr.a[i][s][e >> 2][e & 3];
            b8[e] = (int32_t)fr.b[s][j][e >> 1][e & 1];
        }
        // (operands swapped: B's format goes in the first field)
        if (s == 0) {
            const Acc zero = {};
            blk[j] = F::template mma<FB, FA>(b8, a8, zero);
        } else {
            blk[j] = F::template mma<FB, FA>(b8, a8, blk[j]);
        }
    };
    auto promote = [&](int i, int j) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = __builtin_fmaf(blk[j][r], f[i], acc[i][j][r]);
    };
    u32x2 sap;
    float sbv;
    auto read_scales = [&](auto STG) __attribute__((always_inline)) {
        constexpr uint32_t so = decltype(STG)::value * 1024;
        sap = *reinterpret_cast<const MPDT_LDS u32x2*>(lds0 + lsa + so);
        sbv = *reinterpret_cast<const MPDT_LDS float*>(lds0 + lsb + so);
    };
    auto make_f = [&](int i) __attribute__((always_inline)) {
        if constexpr (ROWS) {
            f[i] = 1.0f;
        } else {
            const uint32_t sa = sap[i];
            f[i] = __uint_as_float(sa) * sbv;
        }
    };

    // Slots 0..7 of K tile t in stage S: promotions of the previous tile's row
    // tile 1 in slots 0-3; the last five direct loads of tile t-1+NS (into
    // stage S-1) in slots 0-4; tile t's remaining fragments in slots 2, 5 and
    // 6 (their registers were last used in slots 11-15 of tile t-1), its row
    // tile 1 multiplier in slot 4 (the previous one was last used in slot 3);
    // the resources of tile t+NS in slot 5.
    auto phase_x = [&](auto STG, bool live_next) __attribute__((always_inline)) {
        using PREV = std::integral_constant<int, (decltype(STG)::value + NS - 1) % NS>;
        static_for<0, 8>([&](auto N) __attribute__((always_inline)) {
            constexpr int n = decltype(N)::value;
            if constexpr (n < 4) promote(1, n);
            mfma(n);
            if constexpr (n <= 4) dma_piece(std::integral_constant<int, 8 + n>{}, rs, PREV{});
            if constexpr (n == 2) rdB(1, 3, STG);
            if constexpr (n == 4) make_f(1);
            if constexpr (n == 5) { rdA(1, 0, STG); rs_next(live_next); }
            if constexpr (n == 6) rdA(1, 1, STG);
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    // Slots 8..15 of a K tile in stage S that is followed by another: the
    // barrier, promotions of row tile 0 in slots 8-11; one direct load of
    // tile t+NS into stage S per slot (the first eight of its 13: a direct
    // load occupies the CU's address unit for 16 cycles, so four waves
    // issuing one per 64-cycle MFMA slot keep it just below saturation); the
    // reads of tile t+1's scales and its fragments for slots 0-7 from stage
    // S+1, each in the slot after the last use of the registers it fills (one
    // B column tile per slot: a burst of reads backs up the LDS queue and
    // stalls the MFMAs that wait for it).
    auto phase_y = [&](auto STG) __attribute__((always_inline)) {
        constexpr int S = decltype(STG)::value;
        using NXT = std::integral_constant<int, (S + 1) % NS>;
        wait_vmem<WAIT_AHEAD>();
        wait_lds();
        wg_barrier();
        static_for<8, 16>([&](auto N) __attribute__((always_inline)) {
            constexpr int n = decltype(N)::value;
            if constexpr (n < 12) promote(0, n - 8);
            mfma(n);
            dma_piece(std::integral_constant<int, n - 8>{}, rs, STG);
            if constexpr (n == 8) { read_scales(NXT{}); rdA(0, 0, NXT{}); }
            if constexpr (n >= 9 && n <= 12) rdB(0, n - 9, NXT{});
            if constexpr (n == 12) rdA(0, 1, NXT{});
            if constexpr (n == 13) rdB(1, 0, NXT{});
            if constexpr (n == 14) { rdB(1, 1, NXT{}); make_f(0); }
            if constexpr (n == 15) rdB(1, 2, NXT{});
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    auto last_tile = [&](auto STG) __attribute__((always_inline)) {
        phase_x(STG, false);
        static_for<8, 16>([&](auto N) __attribute__((always_inline)) {
            constexpr int n = decltype(N)::value;
            if constexpr (n < 12) promote(0, n - 8);
            mfma(n);
            __builtin_amdgcn_sched_barrier(0);
        });
#pragma unroll
        for (int j = 0; j < 4; ++j) promote(1, j);
    };

    // ---- prologue: tiles 0..NS-1 into stages 0..NS-1 (the last five loads of
    // tile NS-1 are issued by tile 0's slots 0-4, as in the steady state) ---
    static_for<0, NS>([&](auto P) __attribute__((always_inline)) {
        if constexpr (decltype(P)::value > 0) rs_next(true);
        constexpr int np = decltype(P)::value == NS - 1 ? 8 : DMA_PER_TILE;
        static_for<0, np>([&](auto Q) __attribute__((always_inline)) { dma_piece(Q, rs, P); });
    });
    wait_vmem<(NS - 2) * DMA_PER_TILE + 8>();
    wg_barrier();
    // what a previous tile's slots 12..15 would have read and computed
    using I0 = std::integral_constant<int, 0>;
    read_scales(I0{});
    rdA(0, 0, I0{});
#pragma unroll
    for (int j = 0; j < 4; ++j) rdB(0, j, I0{});
    rdA(0, 1, I0{});
#pragma unroll
    for (int j = 0; j < 3; ++j) rdB(1, j, I0{});
    make_f(0);

    // ---- K loop, unrolled by NS (stage of tile t = t % NS) ------------------
    int t = 0;
    for (; t + NS <= nt - 1; t += NS) {
        static_for<0, NS>([&](auto S) __attribute__((always_inline)) {
            phase_x(S, t + decltype(S)::value + NS < nt);
            phase_y(S);
        });
    }
    static_for<0, NS - 1>([&](auto S) __attribute__((always_inline)) {
        if (t < nt - 1) {
            phase_x(S, t + NS < nt);
            phase_y(S);
            ++t;
        }
    });
    // t == nt - 1: the last tile, in stage t % NS
    const int sl = t % NS;
    if (sl == 0) last_tile(std::integral_constant<int, 0>{});
    else if (sl == 1) last_tile(std::integral_constant<int, 1>{});
    else last_tile(std::integral_constant<int, (NS > 2 ? 2 : 1)>{});
    // the empty-range loads of the last tiles still write (zeros) to LDS
    wait_vmem<0>();

    MPDT_STAMP(1)
    // ---- epilogue: BF16 D through LDS, 16-byte stores -----------------------
    // A lane holds row i*32 + lrow of the wave tile and, in register 4*r4 + q,
    // column j*32 + 8*r4 + 4*lhalf + q: four consecutive columns per r4, one
    // 8-byte LDS write.  Each wave stages its 64 x 128 tile row-major (256
    // bytes per row, 16-byte chunks XOR-swizzled by row) and writes it out in
    // 16-byte pieces of whole rows.  The LDS serves 128 bytes (32 banks of
    // 4 bytes) per pass, 16 lanes of an 8-byte write: rows r and r + 8 of
    // those 16 lanes share a chunk position modulo 8, so rows whose bit 3 is
    // set keep the two 8-byte halves of a chunk in swapped places and the 16
    // lanes cover all 32 banks once (no conflict); the reads swap them back.
    if constexpr (ROWS) {
        // one scale per row of A and per column of B (increments ld_sa,
        // ld_sb: 1, or 0 for one scale per tensor); full tiles only here
        float sa[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) sa[i] = g.sA[(int64_t)(m0 + wm * C::WM + i * 32 + (int)lrow) * g.ld_sa];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int col = n0 + wn * C::WN + j * 32 + 8 * (r >> 2) + 4 * (int)lhalf + (r & 3);
                const float sb = g.sB[(int64_t)col * g.ld_sb];
#pragma unroll
                for (int i = 0; i < 2; ++i) acc[i][j][r] = (acc[i][j][r] * sa[i]) * sb;
            }
    }
    wg_barrier();   // every wave is past its reads of the K-tile stages
    MPDT_LDS char* const reg = lds0 + wave * (C::WM * C::WN * 2);
    static_assert(4 * C::WM * C::WN * 2 <= LDS_TOTAL, "epilogue staging fits");
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
                *reinterpret_cast<MPDT_LDS u32x2*>(reg + row * 256 + ((c ^ (row & 15)) << 4) +
                                                   8 * (lhalf ^ ((row >> 3) & 1))) = v;
            }
    uint16_t* const dbase = (uint16_t*)g.D + (int64_t)(m0 + wm * C::WM) * g.ldd + n0 + wn * C::WN;
    const bool d_lines = ((uintptr_t)g.D % 128 == 0) && ((g.ldd * 2) % 128 == 0);
    // rows from row_lo and 8-column pieces left of N (N is a multiple of 16);
    // the tile's place is worked out again here rather than kept through the
    // K loop, where every register is taken
    // (row-scaled problems come here with full tiles only)
    int row_skip = 0, cols_left = C::WN;
    if constexpr (!ROWS) {
        int wg = blockIdx.x, etm, etn;
        asm volatile("" : "+s"(wg));
        tile_of(wg, g.tiles_m, g.tiles_n, etm, etn);
        row_skip = etm * C::BM - (m0 + wm * C::WM);
        cols_left = g.N - (etn * C::BN + wn * C::WN);
    }
    if constexpr (ROWS) {
#pragma unroll 4
        for (int q = 0; q < C::WM * 16 / 64; ++q) {
            const int idx = q * 64 + lane;
            const int row = idx >> 4, c = idx & 15;
            u32x4 v = lds_load16(reg, (uint32_t)(row * 256 + ((c ^ (row & 15)) << 4)));
            if ((row >> 3) & 1) v = u32x4{v[2], v[3], v[0], v[1]};
            // D is written once: non-temporal stores when its rows start on
            // 128-byte lines (streamed partial lines cost more than they save)
            u32x4* const dq = reinterpret_cast<u32x4*>(dbase + (int64_t)row * g.ldd + c * 8);
            if (d_lines) __builtin_nontemporal_store(v, dq);
            else *dq = v;
        }
    } else {
        // Buffer stores over the wave's 64 rows of D: a lane whose piece is
        // above row_lo or at or past N gets an offset past the range, and its
        // store is dropped (no branch around the stores).
        const __amdgpu_buffer_rsrc_t drs = buffer_rsrc(dbase, (uint32_t)(C::WM * 2) * (uint32_t)g.ldd);
#pragma unroll 4
        for (int q = 0; q < C::WM * 16 / 64; ++q) {
            const int idx = q * 64 + lane;
            const int row = idx >> 4, c = idx & 15;
            u32x4 v = lds_load16(reg, (uint32_t)(row * 256 + ((c ^ (row & 15)) << 4)));
            if ((row >> 3) & 1) v = u32x4{v[2], v[3], v[0], v[1]};
            const uint32_t off = (row >= row_skip && c * 8 < cols_left)
                                     ? ((uint32_t)row * (uint32_t)g.ldd + (uint32_t)(c * 8)) * 2u
                                     : 0x80000000u;
            // D is written once: non-temporal stores when its rows start on
            // 128-byte lines (streamed partial lines cost more than they save)
            if (d_lines) __builtin_amdgcn_raw_buffer_store_b128(v, drs, off, 0, 2 /* nt */);
            else __builtin_amdgcn_raw_buffer_store_b128(v, drs, off, 0, 0);
        }
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

int fp8_1w_mode(const GemmArgs& a, bool aligned) {
    using C = CfgFP8W;
    const bool full = aligned && a.K % C::KT_BYTES == 0 && a.K >= C::STAGES * C::KT_BYTES &&
                      a.lda_b < (int64_t(1) << 31) / C::BM && a.ldb_b < (int64_t(1) << 31) / C::KROWS &&
                      a.ld_sa < (int64_t(1) << 31) / (4 * C::WM) && ((uintptr_t)a.D % 16) == 0 &&
                      a.ldd % 8 == 0 && a.ldd < (int64_t(1) << 31) / (2 * C::WM);
    // (B rows of at least 256 bytes: the scalar offsets of the B pieces,
    // K-row offsets less the 1 KiB steps of the instruction offset, stay
    // non-negative)
    if (!full || a.ldb_b < C::B_ROW) return 0;
    // (the row-scaled variants take full tiles only: their epilogue leaves
    // no registers for the edge masks)
    return (a.M >= C::BM && a.N % 16 == 0 && !a.row_scaled) ? 2 : 1;
}

template <int F8>
static hipError_t launch_fp8_1w_t(const GemmArgs& a, hipStream_t stream) {
    using C = CfgFP8W;
    hipLaunchKernelGGL((gemm_fp8_1w_kernel<C, F8>), dim3((unsigned)(a.tiles_m * a.tiles_n)), dim3(C::NT),
                       0, stream, a);
    return hipGetLastError();
}

hipError_t launch_fp8_1w(const GemmArgs& a0, int tiles_m, int tiles_n, hipStream_t stream) {
    GemmArgs a = a0;
    a.tiles_m = tiles_m;
    a.tiles_n = tiles_n;
    a.int_tm = a.int_tn = 0;
    switch (fp8_variant(a)) {
        case 0: return launch_fp8_1w_t<0>(a, stream);
        case 1: return launch_fp8_1w_t<1>(a, stream);
        case 2: return launch_fp8_1w_t<2>(a, stream);
        case 3: return launch_fp8_1w_t<3>(a, stream);
        case 4: return launch_fp8_1w_t<4>(a, stream);
        case 5: return launch_fp8_1w_t<5>(a, stream);
        case 6: return launch_fp8_1w_t<6>(a, stream);
        case 7: return launch_fp8_1w_t<7>(a, stream);
    }
    return hipErrorInvalidValue;
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
