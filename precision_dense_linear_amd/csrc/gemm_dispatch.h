// Tile-class dispatch of the per-tensor and grouped FP8 GEMM, for one
// operand-format pair FMT (bit 0: A holds E5M2 codes, bit 1: B; else E4M3).
// Each format pair is instantiated in a translation unit of its own
// (gemm.hip, gemm_fmt1.hip, gemm_fmt2.hip, gemm_fmt3.hip).
#pragma once

#include "gemm_kernel.h"

namespace fp8k {

// Split choice (gemm.hip).  A split tile of the workspace holds the FP32
// partial sums of one 32 x 64 tile (SPLIT_TILE_FLOATS floats).
constexpr int64_t SPLIT_TILE_FLOATS = 32 * 64;
int64_t split_slots();
int choose_splits(int64_t tiles, int64_t K, int per_cu, int64_t capacity);

inline int64_t tiles_of(int64_t M, int64_t N, int BM, int BN) { return ((M + BM - 1) / BM) * ((N + BN - 1) / BN); }

// Plain GEMM with M <= 16 (gemm_skinny.hip): the split count it would use
// (0 when the skinny class does not take the problem), and the launch.
int skinny_splits(const GemmProblem& g);
template <int FMT>
hipError_t launch_skinny(const GemmProblem& g, hipStream_t s, int splits);

template <int FMT, int BM, int BN, int WM, int WN, int KS, int NB, int GROUP_M>
hipError_t launch_cfg(const GemmProblem& g, hipStream_t s) {
    return g.fast_acc ? launch_mode<BM, BN, WM, WN, KS, NB, GROUP_M, MODE_FAST, false, FMT>(g, s)
                      : launch_mode<BM, BN, WM, WN, KS, NB, GROUP_M, MODE_EXACT, false, FMT>(g, s);
}

// The same tile class with K split `splits` ways across workgroups, their
// partials in the caller's workspace (tiles * splits <= its split tiles).
template <int FMT, int BM, int BN, int WM, int WN, int KS, int NB, int GROUP_M>
hipError_t launch_cfg_splitk(const GemmProblem& g, hipStream_t s, int32_t splits) {
    static_assert(BM * BN == SPLIT_TILE_FLOATS, "workspace sized for this tile");
    if (tiles_of(g.M, g.N, BM, BN) * splits > g.ws_tiles || !g.ws || !g.counters) return hipErrorInvalidValue;
    float* ws = g.ws;
    uint32_t* counters = g.counters;
    return g.fast_acc
               ? launch_mode<BM, BN, WM, WN, KS, NB, GROUP_M, MODE_FAST, true, FMT>(g, s, splits, ws, counters)
               : launch_mode<BM, BN, WM, WN, KS, NB, GROUP_M, MODE_EXACT, true, FMT>(g, s, splits, ws, counters);
}

// Tile configuration by shape class (a static table, no runtime tuning):
//  * a plain GEMM with M <= 16 whose K the caller's workspace lets the
//    skinny streaming kernel split (or that has enough 256-column tiles to
//    fill half the CUs unsplit): that kernel (gemm_skinny.hip), in either
//    accumulation mode -- reading B bounds it, so the exact products cost
//    nothing over the FP8 rate;
//  * M (rows per expert when grouped) <= 64: 32 x 64 tiles with each K step
//    split over two wave groups -- many workgroups to stream B, HBM bound; a
//    plain GEMM with fewer such tiles than half the GPU's workgroup slots
//    also splits K across workgroups when the caller gave a workspace
//    (measured on M = 16/32, N = 8192, K = 8192 with B out of HBM:
//    36.5 -> 26 us);
//  * M <= 1024: 128 x 128 tiles, 4 waves of 64 x 64 per K half, the K range
//    split over two wave groups (more loads in flight per tile) -- unless a
//    plain GEMM has so few of them that they would fill under half of the
//    CUs: then, if there are more 64 x 64 tiles than half the CUs, those
//    tiles, 2 waves of 64 x 32 per K half, else the 32 x 64 class (measured,
//    kernel time, exact mode: 1024^3 11.8 -> 8.6 us with 32 x 64 tiles and
//    10.4 -> 9.8 us (event-timed) with 64 x 64; 512 x 2048 x 4096 27.0 ->
//    18.6 and 20.4 -> 18.9 us, FP8_ACC_FAST 18.3 -> 14.0 us; 1024 x 1024 x
//    8192 47.6 -> 32.8 and 36.1 -> 31.2 us, FP8_ACC_FAST 32.0 -> 24.9 us: a
//    64-row tile reads A and B once per 64 x 64 outputs, half of B's bytes
//    of a 32-row one, and these shapes are bound by each CU's L2 request
//    rate; at 128 and more 128 x 128 tiles, e.g. 1024 x 2048 x 1024, the
//    128 x 128 class stays faster; with at most half as many 64 x 64 tiles
//    as CUs the 32 x 64 class's twice as many workgroups win: 512 x 1024 x
//    4096 (128 tiles) 14.8 against 17.3 us, 128 x 2048 x 8192 (64) 21.9
//    against 26.8 us, while 768 x 768 x 2048 (144) takes 12.0 against 12.6;
//    for M <= 64 the 32 x 64 class wastes fewer rows: 40 x 4096 x 4096 13.7
//    us against 16.6);
//  * larger M, and a plain GEMM with M <= 1024 whose 256 x 256 tiles fill at
//    least 7/8 of the CUs with at most 1/8 of their rows padding: 256 x 256
//    tiles, 4 waves of 128 x 128 -- MFMA bound (against the 128 x 128
//    class, exact [FP8_ACC_FAST], event-timed: 1024 x 28672 x 8192 439 ->
//    392 us [319 -> 198], 512 x 28672 x 8192 251 -> 212 [139 -> 96],
//    768 x 28672 x 8192 360 -> 352 [212 -> 180]; slower with fewer tiles,
//    1024 x 8192 x 8192 142 -> 169 [71 -> 82], or more padding, 384 x
//    28672 x 8192 189 -> 196).
template <int FMT>
hipError_t launch_gemm_t(const GemmProblem& g, hipStream_t s) {
    const bool plain = g.experts == 0;
    if (plain && g.M <= 16) {
        const int sk = skinny_splits(g);
        if (sk > 0) return launch_skinny<FMT>(g, s, sk);
    }
    const int64_t rows_per_problem = plain ? g.M : (g.M + g.experts - 1) / g.experts;
    // split_slots() is twice the CU count
    const bool few_mid_tiles = plain && tiles_of(g.M, g.N, 128, 128) * 4 < split_slots();
    if (rows_per_problem <= 64 || (rows_per_problem <= 1024 && few_mid_tiles)) {
        const int sp = plain && g.ws_tiles > 0 ? choose_splits(tiles_of(g.M, g.N, 32, 64), g.K, 2, g.ws_tiles) : 1;
        if (sp > 1) return launch_cfg_splitk<FMT, 32, 64, 1, 2, 2, 4, 8>(g, s, sp);
        if (rows_per_problem > 64 && tiles_of(g.M, g.N, 64, 64) * 4 > split_slots())
            return launch_cfg<FMT, 64, 64, 1, 2, 2, 4, 8>(g, s);
        return launch_cfg<FMT, 32, 64, 1, 2, 2, 4, 8>(g, s);
    }
    if (rows_per_problem <= 1024) {
        // a plain GEMM whose 256 x 256 tiles fill at least 7/8 of the CUs,
        // with at most 1/8 of their rows padding: the 256 x 256 class
        const int64_t cus = split_slots() / 2, padded = (g.M + 255) / 256 * 256;
        if (plain && tiles_of(g.M, g.N, 256, 256) * 8 >= 7 * cus && 8 * (padded - g.M) <= g.M)
            return launch_cfg<FMT, 256, 256, 2, 2, 1, 4, 8>(g, s);
        return launch_cfg<FMT, 128, 128, 2, 2, 2, 4, 8>(g, s);
    }
    return launch_cfg<FMT, 256, 256, 2, 2, 1, 4, 8>(g, s);
}

}  // namespace fp8k
