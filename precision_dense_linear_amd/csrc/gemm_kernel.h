// The FP8 GEMM tile loop for gfx950, instantiated by gemm.hip (per-tensor
// and grouped GEMM: MODE_FAST, MODE_EXACT) and gemm_blockscaled.hip
// (MODE_BLOCK, MODE_BLOCK64).
//
//   C[m, n] = (scale_a * scale_b) * sum_k A[m, k] * B[k, n]
//
// E4M3 (or E5M2) operands, FP32 accumulation, the scales applied once to
// the finished sum, FP32, BF16 or FP16 (RNE) output ("Triton FP8 GEMM via
// CUTLASS naming": kernel
// section, the paragraph after it and the parameter list).  A is M x K with K
// contiguous and B is K x N with N contiguous, as in the kernel sketch of
// "FP8 GEMM in JAX with Triton for Blackwell"; the grouped form runs the same
// tile loop over expert row ranges with per-expert scales (that page's MoE
// paragraph).
//
// The block-scaled form (32x32 tile scales, the parameter paragraph of "FP8
// GEMM in JAX with Triton for Blackwell"; 64x64 tiles, the coarser
// granularity of its monitoring paragraph) runs the same tile loop and folds
// each 32- or 64-deep K block's partial product into the FP32 accumulator
// with its scale pair (the promotion step that page assigns to the CUDA
// cores).
//
// Operand feed per 64-byte K slice: lane l (row or column l%32 of its 32-wide
// block, lane group h = l/32) holds the 16-byte K chunks h and h+2 of the
// slice, i.e. K 16h..16h+15 and 32+16h..32+16h+15:
//  * A: two ds_read_b128 from the swizzled A stage;
//  * B: four ds_read_b64_tr_b8, each gathering 8 K-consecutive bytes of one
//    column from the N-contiguous B stage (the 16 lanes of a group address 8
//    K-rows x two 8-byte column halves; lane 8g+c receives column c of half g).
// The 8-byte pieces 0..3 of a lane's 32 bytes thus hold K 16h+8p' + 32p''
// (piece 2p''+p'), so pieces 0-1 of both lane groups cover K 0..31 and
// pieces 2-3 cover K 32..63: one FP8 MFMA (K=64) takes all four -- the
// instruction's own K order, so its 32-deep scale blocks (MODE_E8M0) are
// K 0..31 and 32..63 of the slice -- and the
// K=16 BF16 MFMA fed by piece p stays inside one 32-deep K block.
#pragma once

#include "gemm_common.h"
#include "launch.h"

namespace fp8k {

namespace {

// Operand fragments of one 64-byte K slice for a wave: per A block the two
// 16-byte halves of each lane's 32 bytes, per B block the four 8-byte
// transposed reads.
template <int TM, int TN>
struct Frags {
    v4i a[TM][2];
    v2i b[TN][4];
    int idx[TN];  // MODE_SPARSE: the 2-bit positions of the B block's kept values
};

// Compile-time loop: f(integral_constant<int, I>) for I = 0 .. N-1.
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

// Matrix-core modes of the tile loop.
enum Mode : int {
    MODE_FAST = 0,   // native FP8 MFMA (K=64)
    MODE_EXACT = 1,  // E4M3 widened exactly to BF16, K=16 BF16 MFMAs
    MODE_BLOCK = 2,    // as MODE_EXACT, with a scale pair per 32x32 block and 32-deep K block
    MODE_BLOCK64 = 3,  // the same with 64x64 scale tiles and 64-deep K blocks (one per slice)
    MODE_E8M0 = 4,     // native FP8 MFMA with a power-of-two (E8M0) scale per 32x32 tile of A and of B,
                       // applied by the matrix core to each 32-deep K block
    MODE_SPARSE = 5,   // 2:4-sparse B (compressed values + 2-bit positions) on the sparse FP8 MFMA
};

// FMT: operand formats, bit 0 set = A holds E5M2 codes, bit 1 = B (else E4M3).
template <int BM, int BN, int WM, int WN, int KS, int NB, int GROUP_M, bool BF16, int MODE, bool SPLITK = false,
          int FMT = 0>
__global__ void __launch_bounds__(64 * WM * WN * KS) gemm_kernel(GemmArgs p) {
    constexpr bool BLOCKED = MODE == MODE_BLOCK || MODE == MODE_BLOCK64;
    constexpr int KBD = MODE == MODE_BLOCK64 ? 64 : 32;  // K depth and edge of a scale tile
    constexpr int KB_PER_SLICE = BKP / KBD;             // scale blocks per 64-byte slice: 2 or 1
    static_assert(!BLOCKED || FMT == 0, "the block-scaled form takes E4M3 operands");
    constexpr bool E8 = MODE == MODE_E8M0;
    constexpr bool SP = MODE == MODE_SPARSE;
    static_assert(!SP || (FMT == 0 && KS == 1 && !SPLITK), "sparse B: E4M3, one wave group, no split-K");
    static_assert(!E8 || (FMT == 0 && KS == 1), "E8M0 tile scales: E4M3 operands, whole K blocks per wave");
    constexpr int FA = FMT & 1, FB = (FMT >> 1) & 1;
    using C = PipeCfg<BM, BN, WM, WN, KS, NB, SP>;
    constexpr int TM = C::TM, TN = C::TN;
    constexpr bool WIDEN = MODE != MODE_FAST && !E8 && !SP;
    static_assert(!BLOCKED || KS == 1, "block scales need whole K blocks per wave group");
    // The configurations the dispatch uses and the tests cover; one wave
    // group with 32 x 32 wave tiles (e.g. 64 x 64 tiles of 2 x 2 waves) gave
    // wrong results in a trial build and is not supported.
    static_assert(KS > 1 || (TM >= 2 && TN >= 2), "one wave group needs wave tiles of at least 64 x 64");
    static_assert(MODE != MODE_BLOCK64 || (C::WTM % 64 == 0 && C::WTN % 64 == 0),
                  "a wave tile covers whole 64x64 scale tiles");
    constexpr int EPI = (KS > 1 ? C::RED : 0) + WM * WN * TileStore<BF16, TM, TN>::LDS_BYTES;
    static_assert(EPI <= 160 * 1024, "epilogue LDS budget");
    __shared__ __attribute__((aligned(1024))) uint8_t smem[C::LDS > EPI ? C::LDS : EPI];

    const TileSlice t = resolve_tile<BM, BN, GROUP_M>(p);
    if (!t.valid) return;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ks = wave / (WM * WN);
    const int wm = (wave % (WM * WN)) / WN;
    const int wn = wave % WN;
    const int64_t K = p.K, N = p.N;
    // This workgroup's K range: whole A stages (KS * 128 bytes of K), dealt
    // over the splits of the tile as evenly as they divide (all of K without
    // split-K; never an empty range while splits <= stages).
    const int64_t kstep = KS * BKA;
    const int64_t nkst = (K + kstep - 1) / kstep;
    const int64_t k_begin = min<int64_t>(t.split * nkst / p.splits * kstep, K);
    const int64_t k_end = min<int64_t>((t.split + 1) * nkst / p.splits * kstep, K);
    // slices per wave group: whole A stages
    const int nsteps = 2 * (int)((k_end - k_begin + kstep - 1) / kstep);
    lds_u8* lds = (lds_u8*)smem;
    using Loader = PipeLoader<BM, BN, WM, WN, KS, NB, SP>;
    const Loader loader(t, N, K, k_begin, k_end, wave, lane, (uint32_t)(uintptr_t)lds, p.sp_idx);

    v16f acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // Per-lane LDS byte offsets of this wave's operands: A in A stage 0 for
    // both slices u of a stage and both of a lane's 16-byte chunks (chunk
    // 4u + h + 2j of its row, at its XOR position), B in B stage 0 (B stage j
    // adds the constant j * B_STAGE).
    const int h = lane >> 5;
    int a_off[2][TM][2];
    int b_off[TN][4];
#pragma unroll
    for (int mi = 0; mi < TM; ++mi) {
        const int row = wm * C::WTM + mi * 32 + (lane & 31);
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                a_off[u][mi][j] = ks * BM * BKA + row * BKA + swz_a128(row, 4 * u + h + 2 * j) * 16;
    }
#pragma unroll
    for (int ni = 0; ni < TN; ++ni) {
        const int col = wn * C::WTN + ni * 32 + 16 * ((lane >> 4) & 1) + 8 * (lane & 1);
#pragma unroll
        for (int tq = 0; tq < 4; ++tq) {
            // SP: pieces 0, 1 are compressed rows 16h .. 16h+15 (the kept values of K 32h .. 32h+31)
            const int kr = SP ? 16 * h + 8 * (tq & 1) + ((lane & 15) >> 1)
                              : 16 * h + 8 * (tq & 1) + 32 * (tq >> 1) + ((lane & 15) >> 1);
            b_off[ni][tq] = C::B_BASE + ks * BKP * BN + kr * BN + swz_b<BN>(kr, col >> 4) * 16 + (col & 15);
        }
    }
    // SP: the index word of K block 2s + h for this lane's column of B block ni
    int idx_off[TN];
#pragma unroll
    for (int ni = 0; ni < TN; ++ni) idx_off[ni] = C::B_BASE + C::B_VAL + h * BN * 4 + (wn * C::WTN + ni * 32 + (lane & 31)) * 4;

    // A slice's LDS reads in a fixed order: q < 2*TM reads chunk q%2 of A
    // block q/2, the rest read piece (q-2TM)%PB of B block (q-2TM)/PB (PB = 4
    // pieces, or 2 of compressed values in MODE_SPARSE, followed there by the
    // TN index words).  `abuf` is the LDS address of the slice's A stage; U
    // (slice within the A stage) and BB (B stage buffer) are compile-time.
    constexpr int PB = SP ? 2 : 4;
    constexpr int RD = 2 * TM + PB * TN + (SP ? TN : 0);
    auto read_one = [&](auto q_c, auto u_c, auto bb_c, const lds_u8* abuf, Frags<TM, TN>& f) {
        constexpr int q = decltype(q_c)::value, u = decltype(u_c)::value, bb = decltype(bb_c)::value;
        if constexpr (q < 2 * TM) {
            f.a[q / 2][q % 2] = lds_read16(abuf + a_off[u][q / 2][q % 2]);
        } else if constexpr (q < 2 * TM + PB * TN) {
            constexpr int qb = q - 2 * TM;
            f.b[qb / PB][qb % PB] = lds_read_tr8(lds + bb * C::B_STAGE + b_off[qb / PB][qb % PB]);
        } else {
            constexpr int qi = q - 2 * TM - PB * TN;
            f.idx[qi] = *(const __attribute__((address_space(3))) int*)(lds + bb * C::B_STAGE + idx_off[qi]);
        }
    };
    auto a_op = [](const Frags<TM, TN>& f, int mi) {
        const v4i lo = f.a[mi][0], hi = f.a[mi][1];
        return (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
    auto b_op = [](const Frags<TM, TN>& f, int ni) {
        return (v8i){f.b[ni][0][0], f.b[ni][0][1], f.b[ni][1][0], f.b[ni][1][1],
                     f.b[ni][2][0], f.b[ni][2][1], f.b[ni][3][0], f.b[ni][3][1]};
    };
    auto b_sparse_op = [](const Frags<TM, TN>& f, int ni) {  // 16 compressed values: K 32h .. 32h+31
        return (v4i){f.b[ni][0][0], f.b[ni][0][1], f.b[ni][1][0], f.b[ni][1][1]};
    };

    // The slice's matrix instructions in a fixed order.  Fast: one K=64 FP8
    // MFMA per block, index (mi, ni).  Widened modes: four K=16 BF16 MFMAs
    // per block; piece c of each lane's bytes (for A and B alike) feeds MFMAs
    // c*TM*TN .. +TM*TN-1, piece-outermost so consecutive MFMAs update
    // different accumulators.  The B fragment is the first operand, so
    // accumulator block (mi, ni) holds C^T (see TileStore).
    constexpr int BLK = TM * TN;
    constexpr int MF = BLK * (WIDEN ? 4 : 1);
    v8bf ab[2][TM], bb[2][TN];  // widened modes: piece c as BF16 in set c & 1
    auto convert = [&](auto c_c, const Frags<TM, TN>& f) {
        constexpr int c = decltype(c_c)::value;
#pragma unroll
        for (int mi = 0; mi < TM; ++mi)
            ab[c & 1][mi] = fp8x8_to_bf16<FA>(f.a[mi][c / 2][(c % 2) * 2], f.a[mi][c / 2][(c % 2) * 2 + 1]);
#pragma unroll
        for (int ni = 0; ni < TN; ++ni) bb[c & 1][ni] = fp8x8_to_bf16<FB>(f.b[ni][c][0], f.b[ni][c][1]);
    };
    // Block modes: the K block's partial product per accumulator block
    // (pieces 2kb and 2kb+1 of the slice for 32-deep blocks, all four pieces
    // for 64-deep ones), folded into acc with its scale.
    v16f part[BLOCKED ? TM : 1][BLOCKED ? TN : 1];
    // MODE_E8M0: this slice's scale operands, per lane: byte mi (ni) holds
    // the exponent of A block mi (B block ni) for K block 2s + h (the scaled
    // MFMA takes the exponent of 32-deep K block b of a row or column from
    // lane group b), selected per MFMA by its op_sel field.
    int e8a_lane = 0, e8b_lane = 0;
    auto mfma_one = [&](auto m_c, const Frags<TM, TN>& f) {
        constexpr int m = decltype(m_c)::value;
        if constexpr (MODE == MODE_EXACT) {
            constexpr int c = m / BLK, mi = (m % BLK) / TN, ni = m % TN;
            acc[mi][ni] = mfma_32x32x16_bf16(bb[c & 1][ni], ab[c & 1][mi], acc[mi][ni]);
        } else if constexpr (BLOCKED) {
            constexpr int c = m / BLK, mi = (m % BLK) / TN, ni = m % TN;
            const v16f zero = {};
            constexpr bool first = MODE == MODE_BLOCK ? (c % 2 == 0) : (c == 0);  // first piece of its K block
            part[mi][ni] = mfma_32x32x16_bf16(bb[c & 1][ni], ab[c & 1][mi], first ? zero : part[mi][ni]);
        } else if constexpr (SP) {
            constexpr int mi = m / TN, ni = m % TN;
            acc[mi][ni] = smfmac_32x32x64_e4m3(b_sparse_op(f, ni), a_op(f, mi), acc[mi][ni], f.idx[ni]);
        } else if constexpr (E8) {
            constexpr int mi = m / TN, ni = m % TN;
            acc[mi][ni] = mfma_32x32x64_e4m3_scaled<ni, mi>(b_op(f, ni), a_op(f, mi), acc[mi][ni], e8b_lane, e8a_lane);
        } else {
            constexpr int mi = m / TN, ni = m % TN;
            acc[mi][ni] = mfma_32x32x64_f8<FB, FA>(b_op(f, ni), a_op(f, mi), acc[mi][ni]);
        }
    };
    // Block modes' scale indices: tile-scale row of each A block and column
    // of each B block (clamped: blocks past M or N are never stored), and the
    // numbers of KBD-deep K blocks and KBD-wide column blocks.
    int sa_row[TM], sb_col[TN];
    const int64_t KBLK = K / KBD, NBLK = N / KBD;
    if constexpr (BLOCKED || E8) {
#pragma unroll
        for (int mi = 0; mi < TM; ++mi)
            sa_row[mi] = (int)min<int64_t>((t.m0 + wm * C::WTM + mi * 32) / KBD, t.M / KBD - 1);
#pragma unroll
        for (int ni = 0; ni < TN; ++ni)
            sb_col[ni] = (int)min<int64_t>((t.n0 + wn * C::WTN + ni * 32) / KBD, NBLK - 1);
    }
    // (The block modes are launched with K > 0 only: K == 0 has empty scale
    // arrays, and its all-zero C is written by the launchers instead.)
    // Block modes' tile scales: read through the constant address space, so
    // they come in by scalar loads, counted by lgkmcnt rather than by the
    // vmcnt that tracks the stage loads, and one slice ahead, so the
    // lgkmcnt(0) wait at the next slice's barrier covers them.  sa_nx / sb_nx
    // hold the scales of the next slice's K blocks (two 32-deep or one
    // 64-deep; clamped: past the end of K the partial products are zero).
    typedef const __attribute__((address_space(4))) float cfloat;
    float sa_nx[2][TM], sb_nx[2][TN];
    auto load_slice_scales = [&](int64_t sl) {
#pragma unroll
        for (int r = 0; r < KB_PER_SLICE; ++r) {
            const int64_t k = min<int64_t>(KB_PER_SLICE * sl + r, KBLK - 1);
#pragma unroll
            for (int mi = 0; mi < TM; ++mi) sa_nx[r][mi] = *(cfloat*)(p.scale_a + sa_row[mi] * KBLK + k);
#pragma unroll
            for (int ni = 0; ni < TN; ++ni) sb_nx[r][ni] = *(cfloat*)(p.scale_b + k * NBLK + sb_col[ni]);
        }
    };
    // MODE_E8M0 tile exponents: the K-block-major byte arrays e8_a
    // [K/32][pitch_a] and e8_b [K/32][pitch_b], each row padded to a
    // multiple of 4 bytes, so that the TM (TN) consecutive row (column)
    // tiles of a wave (TM, TN = 2 or 4, starting at a multiple of TM / TN)
    // lie in one aligned 4-byte word per K block, at a byte shift fixed per
    // wave.  Read through the constant address space (scalar loads, like the
    // block scales above) one slice ahead.
    typedef const __attribute__((address_space(4))) uint32_t cuint;
    const uint32_t pitch_a = (uint32_t)((((t.M + 31) / 32) + 3) & ~3);
    const uint32_t pitch_b = (uint32_t)((NBLK + 3) & ~3);
    // first tile of the wave (clamped: a wave wholly past M or N stores
    // nothing, but its reads must stay inside the arrays)
    const uint32_t e8a_t0 = (uint32_t)min<int64_t>((t.m0 + wm * C::WTM) / 32, (t.M + 31) / 32 - 1);
    const uint32_t e8b_t0 = (uint32_t)min<int64_t>((t.n0 + wn * C::WTN) / 32, NBLK - 1);
    const uint32_t e8a_sh = 8 * (e8a_t0 & 3), e8b_sh = 8 * (e8b_t0 & 3);
    uint32_t e8a_w[2], e8b_w[2];  // words of the next slice's K blocks 2s, 2s+1
    auto load_slice_e8 = [&](int64_t sl) {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const uint32_t k = (uint32_t)min<int64_t>(2 * sl + r, KBLK - 1);
            e8a_w[r] = *(cuint*)(p.e8_a + (k * pitch_a + (e8a_t0 & ~3u)));
            e8b_w[r] = *(cuint*)(p.e8_b + (k * pitch_b + (e8b_t0 & ~3u)));
        }
    };
    // acc += s_a * s_b * part for every accumulator block, with the scales
    // (sa, sb) of the K block just multiplied
    auto fold = [&](const float (&sa)[TM], const float (&sb)[TN]) {
#pragma unroll
        for (int mi = 0; mi < TM; ++mi)
#pragma unroll
            for (int ni = 0; ni < TN; ++ni) {
                const float sc = sa[mi] * sb[ni];
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[mi][ni][r] = fmaf(sc, part[mi][ni][r], acc[mi][ni][r]);
            }
    };

    // Pipeline (load schedule in PipeLoader).  Slice s, whose fragments are
    // already in registers or requested:
    //   wait until the loads of slice s-NB+1 and earlier have landed (the
    //   later NB-2 slices' loads may still be in flight) and this wave's LDS reads
    //   are complete; barrier -- the stages that slice s+1 reads are visible to
    //   all waves, and no wave still reads the buffers slice s refills;
    //   then G regions, each: a share of the slice s+1 LDS reads, a share of
    //   the slice s MFMAs, and a share of the slice's LPS loads.
    // Spreading the loads between the MFMAs keeps the four waves from
    // queueing a whole stage of loads at once behind the barrier, which
    // stalls each wave's MFMA issue until the address unit has accepted them.
    // In the block modes a region is half a slice (one 32-deep K block, or
    // half of a 64-deep one): its MFMAs, then the fold at the end of each K
    // block.
    // Loads past the end of K are empty (they read zero), so the body is
    // branch-free and the in-flight load count is the same every slice.  The
    // loop is unrolled over the NB B buffers (and fragment register pairs);
    // the slice count is a whole number of A stages, and rounded up to whole
    // loop bodies, the extra slices multiplying zeros (an accumulator that
    // starts at +0 stays exact under +0 terms).
    constexpr int G = BLOCKED ? 2 : C::LPS;  // regions per slice
    constexpr int U = NB;                               // slices per unrolled body
    static_assert(U % 2 == 0, "fragment register pairs and A-stage halves alternate");
    Frags<TM, TN> f0, f1;
    if constexpr (BLOCKED) load_slice_scales(0);
    if constexpr (E8) load_slice_e8(0);
    loader.issue_a_half(-NB - 1);
#pragma unroll
    for (int s = -NB; s < 0; ++s) loader.issue_slice(s);
    wait_vmcnt_lds<(NB - 1) * C::LPS>();
    __syncthreads();
    static_for<0, RD>([&](auto q_c) {
        read_one(q_c, std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{}, lds, f0);
    });

    for (int s0 = 0; s0 < nsteps; s0 += U) {
        static_for<0, U>([&](auto i_c) {
            constexpr int i = decltype(i_c)::value;
            const int s = s0 + i;
            const Frags<TM, TN>& cur = (i & 1) ? f1 : f0;
            Frags<TM, TN>& next = (i & 1) ? f0 : f1;
            wait_vmcnt_lds<(NB - 2) * C::LPS>();
            __syncthreads();
            const typename Loader::Stage stage = loader.prepare(s);
            // block modes: this slice's scales (loaded one slice ago), then
            // the next slice's
            float sa_cur[2][TM], sb_cur[2][TN];
            if constexpr (BLOCKED) {
#pragma unroll
                for (int r = 0; r < KB_PER_SLICE; ++r) {
#pragma unroll
                    for (int mi = 0; mi < TM; ++mi) sa_cur[r][mi] = sa_nx[r][mi];
#pragma unroll
                    for (int ni = 0; ni < TN; ++ni) sb_cur[r][ni] = sb_nx[r][ni];
                }
                load_slice_scales(s + 1);
            }
            if constexpr (E8) {
                e8a_lane = (int)((h ? e8a_w[1] : e8a_w[0]) >> e8a_sh);
                e8b_lane = (int)((h ? e8b_w[1] : e8b_w[0]) >> e8b_sh);
                load_slice_e8(s + 1);
            }
            // slice s+1: A stage (s+1)/2, slice (i+1)&1 of it; B buffer (i+1)%NB
            const lds_u8* abuf = lds + (((s + 1) >> 1) % C::NBUF_A) * C::A_STAGE;
            static_for<0, G>([&](auto r_c) {
                constexpr int r = decltype(r_c)::value;
                constexpr int q0 = RD * r / G, q1 = RD * (r + 1) / G;
                constexpr int m0 = MF * r / G, m1 = MF * (r + 1) / G;
                constexpr int l0 = C::LPS * r / G, l1 = C::LPS * (r + 1) / G;
                if constexpr (MODE == MODE_EXACT) {
                    // widen piece 0 ahead of its MFMAs; piece c >= 1 one region
                    // early (in the region holding MFMA c*BLK - 1), so the
                    // conversions overlap the previous piece's MFMAs
                    if constexpr (r == 0) convert(std::integral_constant<int, 0>{}, cur);
                    static_for<1, 4>([&](auto c_c) {
                        constexpr int c = decltype(c_c)::value;
                        if constexpr (c * BLK - 1 >= m0 && c * BLK - 1 < m1) convert(c_c, cur);
                    });
                }
                static_for<q0, q1>([&](auto q_c) {
                    read_one(q_c, std::integral_constant<int, (i + 1) & 1>{}, std::integral_constant<int, (i + 1) % NB>{},
                             abuf, next);
                });
                constexpr int nq = q1 - q0, nm = m1 - m0;
                if constexpr (BLOCKED) {
                    // pieces 2r and 2r+1 into each block's partial; a K block
                    // ends with this region in MODE_BLOCK (block 2s + r) and
                    // with region 1 in MODE_BLOCK64 (block s): then the fold
                    // of each accumulator block (each depends only on its own
                    // block's last MFMA, so the scheduler can overlap it with
                    // the other blocks' MFMAs)
                    convert(std::integral_constant<int, 2 * r>{}, cur);
                    convert(std::integral_constant<int, 2 * r + 1>{}, cur);
                    static_for<m0, m1>([&](auto m_c) { mfma_one(m_c, cur); });
                    if constexpr (MODE == MODE_BLOCK) fold(sa_cur[r], sb_cur[r]);
                    else if constexpr (r == 1) fold(sa_cur[0], sb_cur[0]);
                } else {
                    static_for<m0, m1>([&](auto m_c) { mfma_one(m_c, cur); });
                }
                // interleave the region's LDS reads with its MFMAs
                if constexpr (!BLOCKED && nm > 0 && nq > 0) {
                    constexpr int RPM = (nq + nm - 1) / nm;
#pragma unroll
                    for (int g = 0; g < (nq + RPM - 1) / RPM; ++g) {
                        __builtin_amdgcn_sched_group_barrier(0x100, RPM, 0);  // DS read
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // MFMA
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
                static_for<l0, l1>([&](auto l_c) { loader.issue_one(stage, decltype(l_c)::value, (i + 1) & 1); });
                __builtin_amdgcn_sched_barrier(0);
            });
        });
    }

    // Drain: the empty tail loads must land before the LDS is reused.
    wait_vmcnt<0>();

    // Split-K: wave groups 1..KS-1 hand their partial sums to group 0 via LDS.
    if constexpr (KS > 1) {
        __syncthreads();
        float* red = (float*)smem;
        const int wslot = wm * WN + wn;
        constexpr int PER = TM * TN * 16 * 64;
        if (ks > 0) {
            float* dst = red + ((ks - 1) * WM * WN + wslot) * PER;
#pragma unroll
            for (int mi = 0; mi < TM; ++mi)
#pragma unroll
                for (int ni = 0; ni < TN; ++ni)
#pragma unroll
                    for (int r = 0; r < 16; ++r) dst[((mi * TN + ni) * 16 + r) * 64 + lane] = acc[mi][ni][r];
        }
        __syncthreads();
#pragma unroll
        for (int g = 0; g < KS - 1; ++g) {
            const float* src = red + (g * WM * WN + wslot) * PER;
#pragma unroll
            for (int mi = 0; mi < TM; ++mi)
#pragma unroll
                for (int ni = 0; ni < TN; ++ni)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[mi][ni][r] += src[((mi * TN + ni) * 16 + r) * 64 + lane];
        }
    }

    // Split-K: every split stores its FP32 partial sums (in the lanes' own
    // layout, coalesced; rows past M skipped) and counts itself in; the last
    // to arrive sums all the tile's partials in split order -- the same order
    // whichever split is last, so the result is deterministic -- and writes
    // C.  Partials, counters and the last split's reads are relaxed
    // device-scope atomics: on gfx950 loads and stores that bypass the
    // non-coherent cache levels (coherent across the XCDs' L2s).  A split
    // counts itself in only after its partial stores have completed (vmcnt
    // 0, then a barrier for the other waves' stores), and the last split
    // reads the partials only after its count has returned; this ordering
    // rests on that cache behaviour rather than on release/acquire, whose
    // whole-L2 write-back and invalidate per workgroup measured 23.8 ->
    // 40.7 us at M = 16, N = K = 8192.  No workgroup ever waits on another.
    // (With KS > 1 only wave group 0 holds the tile's sums; the other groups
    // take part in the barriers and leave before the epilogue.)
    if constexpr (SPLITK) {
        // the flag takes the first LDS word: past the first barrier below no
        // wave reads the stage or reduction buffers any more
        int* last_split = reinterpret_cast<int*>(smem);
        constexpr int PER = TM * TN * 16 * 64;
        const int wslot = wm * WN + wn;
        bool row_ok[TM];
#pragma unroll
        for (int mi = 0; mi < TM; ++mi) row_ok[mi] = t.m0 + wm * C::WTM + mi * 32 + (lane & 31) < t.M;
        float* mine = p.ws + ((int64_t)(t.tile * p.splits + t.split) * (WM * WN) + wslot) * PER;
        if (ks == 0) {
#pragma unroll
            for (int mi = 0; mi < TM; ++mi)
                if (row_ok[mi])
#pragma unroll
                    for (int ni = 0; ni < TN; ++ni)
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            __hip_atomic_store(mine + ((mi * TN + ni) * 16 + r) * 64 + lane, acc[mi][ni][r],
                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        wait_vmcnt<0>();
        __syncthreads();
        if (threadIdx.x == 0)
            *last_split = __hip_atomic_fetch_add(p.counters + t.tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                          (uint32_t)(p.splits - 1);
        __syncthreads();
        if (!*last_split) return;
#pragma unroll
        for (int mi = 0; mi < TM; ++mi)
#pragma unroll
            for (int ni = 0; ni < TN; ++ni)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;
        if (ks == 0) {
            for (int sp = 0; sp < p.splits; ++sp) {
                const float* src = p.ws + ((int64_t)(t.tile * p.splits + sp) * (WM * WN) + wslot) * PER;
#pragma unroll
                for (int mi = 0; mi < TM; ++mi)
                    if (row_ok[mi])
#pragma unroll
                        for (int ni = 0; ni < TN; ++ni)
#pragma unroll
                            for (int r = 0; r < 16; ++r)
                                acc[mi][ni][r] += __hip_atomic_load(src + ((mi * TN + ni) * 16 + r) * 64 + lane,
                                                                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        if (threadIdx.x == 0) __hip_atomic_store(p.counters + t.tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (ks > 0) return;

    // Epilogue: the per-tensor (or per-expert) scales applied once to the
    // sum, one after the other (block scales are already folded in).  With
    // KS > 1 the LDS scratch sits after the reduction buffer; otherwise every
    // wave must first be done with the stage buffers.
    if constexpr (KS == 1) __syncthreads();
    using Store = TileStore<BF16, TM, TN>;
    lds_u8* scratch = lds + (KS > 1 ? C::RED : 0) + (wm * WN + wn) * Store::LDS_BYTES;
    const float sa = (BLOCKED || E8) ? 1.0f : p.scale_a[t.expert];
    const float sb = (BLOCKED || E8) ? 1.0f : p.scale_b[t.expert];
    Store::run(p.C, acc, sa, sb, t.m0 + wm * C::WTM, t.n0 + wn * C::WTN, t.M, N, t.c_row0, lane, scratch,
               p.out_f16 != 0);
}

// Zero `bytes` bytes at p (16-byte aligned; a multiple of 2 bytes): a fill
// kernel rather than a memset, so that a caller may capture it in a graph.
__global__ void fill_zero_kernel(uint8_t* p, int64_t bytes) {
    const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 16;
    if (i + 16 <= bytes) {
        *reinterpret_cast<v4i*>(p + i) = (v4i){0, 0, 0, 0};
    } else {
        for (int64_t j = i; j < bytes; ++j) p[j] = 0;
    }
}

inline hipError_t fill_zero(void* p, int64_t bytes, hipStream_t s) {
    if (bytes <= 0) return hipSuccess;
    const int64_t threads = (bytes + 15) / 16;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
                       reinterpret_cast<uint8_t*>(p), bytes);
    return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, int KS, int NB, int GROUP_M, int MODE, bool SPLITK = false, int FMT = 0>
hipError_t launch_mode(const GemmProblem& g, hipStream_t s, int32_t splits = 1, float* ws = nullptr,
                       uint32_t* counters = nullptr) {
    GemmArgs a;
    a.A = g.A;
    a.B = g.B;
    a.C = g.C;
    a.scale_a = g.scale_a;
    a.scale_b = g.scale_b;
    a.offsets = g.offsets;
    a.experts = g.experts;
    a.M = g.M;
    a.N = g.N;
    a.K = g.K;
    a.tiles_n = (int32_t)((g.N + BN - 1) / BN);
    // grouped: an upper bound of sum_e ceil(rows_e / BM); surplus workgroups exit at once
    a.tiles_m = g.experts == 0 ? (int32_t)((g.M + BM - 1) / BM)
                               : (int32_t)((g.M + (int64_t)g.experts * (BM - 1)) / BM);
    a.splits = SPLITK ? splits : 1;
    a.out_f16 = g.out_f16;
    a.e8_a = g.e8_a;
    a.e8_b = g.e8_b;
    a.sp_idx = g.sp_idx;
    a.ws = ws;
    a.counters = counters;
    const int64_t blocks = (int64_t)a.tiles_m * a.tiles_n * a.splits;
    if (blocks == 0) return hipSuccess;
    constexpr int NT = 64 * WM * WN * KS;
    const dim3 grid((unsigned)blocks), block(NT);
    if (g.out_bf16) hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, KS, NB, GROUP_M, true, MODE, SPLITK, FMT>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, KS, NB, GROUP_M, false, MODE, SPLITK, FMT>), grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace

}  // namespace fp8k
